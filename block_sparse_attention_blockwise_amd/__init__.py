"""Python binding of the MI355X In-context Sparse Attention (ISA) library.

Argument marshalling only: every step of the method runs in the HIP kernels
of libisa_mi355x.so (built from csrc/ for gfx950). PyTorch supplies device
memory and the current HIP stream; the functions below check shapes and
dtypes, allocate outputs and workspace with torch, and call the C entry
points of include/isa.h by the same names. There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libisa_mi355x.so")

ISA_OK = 0
ISA_ERR_ARG = -1
ISA_ERR_UNSUPPORTED = -2
ISA_ERR_WORKSPACE = -3
ISA_ERR_HIP = -4
ISA_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 64 << 20   # ISA_NOALLOC_SCRATCH_BYTES

EXPORTED = ("isa_plan", "isa_pool_coarse", "isa_rope_pool_coarse", "isa_ctx_topk", "isa_sharpness_split",
            "isa_sharp_attn", "isa_flat_taylor_attn", "isa_coarse_residual", "isa_forward",
            "isa_backward", "isa_dense_attn", "isa_forward_noalloc", "isa_init", "isa_strerror")


class IsaParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L_src", ctypes.c_int32),
                ("L_ctx", ctypes.c_int32), ("D", ctypes.c_int32), ("b", ctypes.c_int32),
                ("alpha_s", ctypes.c_double), ("alpha_f", ctypes.c_double),
                ("alpha_ns", ctypes.c_double), ("gamma", ctypes.c_double),
                ("rope_base", ctypes.c_double)]


class IsaPlan(ctypes.Structure):
    _fields_ = [("N_src", ctypes.c_int32), ("N_ctx", ctypes.c_int32), ("N", ctypes.c_int32),
                ("k_ctx", ctypes.c_int32), ("N_kv", ctypes.c_int32), ("n_flat", ctypes.c_int32),
                ("n_sharp", ctypes.c_int32), ("k_ns", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("scores_bytes", ctypes.c_size_t),
                ("rope_bytes", ctypes.c_size_t), ("noalloc_bytes", ctypes.c_size_t)]


class IsaDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("qc", "kc", "ctx_score", "ctx_idx", "sharpness",
                                              "sharp_idx", "flat_idx", "flat_exact_idx")]


class IsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"ISA HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build() or python -m "
                               "block_sparse_attention_blockwise_amd._build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER(IsaParams)
        L.isa_plan.argtypes = [P, ctypes.POINTER(IsaPlan)]
        L.isa_pool_coarse.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.isa_rope_pool_coarse.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.isa_ctx_topk.argtypes = [P, vp, vp, vp, vp, vp]
        L.isa_sharpness_split.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.isa_sharp_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.isa_flat_taylor_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.isa_coarse_residual.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
        L.isa_forward.argtypes = [P, vp, vp, vp, vp, vp, sz, ctypes.POINTER(IsaDebug), vp]
        L.isa_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.isa_dense_attn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.isa_forward_noalloc.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(IsaDebug), vp]
        L.isa_init.argtypes = []
        L.isa_strerror.argtypes = [ctypes.c_int]
        L.isa_strerror.restype = ctypes.c_char_p
        for n in EXPORTED[:-1]:
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().isa_strerror(code).decode()


def _check(fn: str, rc: int):
    if rc != ISA_OK:
        raise IsaError(fn, rc)


@dataclass(frozen=True)
class Params:
    B: int
    H: int
    L_src: int
    L_ctx: int
    D: int
    b: int = 64
    alpha_s: float = 0.125
    alpha_f: float = 0.5
    alpha_ns: float = 0.0625
    gamma: float = 0.0
    rope_base: float = 0.0

    def c(self) -> IsaParams:
        return IsaParams(self.B, self.H, self.L_src, self.L_ctx, self.D, self.b,
                         self.alpha_s, self.alpha_f, self.alpha_ns, self.gamma, self.rope_base)


def plan(p: Params) -> dict:
    """Counts and workspace sizes (host only; no GPU needed)."""
    out = IsaPlan()
    _check("isa_plan", lib().isa_plan(ctypes.byref(p.c()), ctypes.byref(out)))
    return {f: getattr(out, f) for f, _ in IsaPlan._fields_}


# ------------------------------------------------------------- torch glue
# Every tensor handed to the library is checked here (device, dtype,
# contiguity, exact shape): the C entry points receive bare pointers and
# cannot tell a wrong-sized buffer from a right one.
def _torch():
    import torch
    return torch


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _req(name: str, t, shape, dtype, device=None):
    """Raise unless `t` is a contiguous `dtype` tensor of exactly `shape` on
    a HIP device (on `device` when given)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _req_bytes(name: str, t, nbytes: int, device):
    """Raise unless `t` is a contiguous device buffer of at least `nbytes`."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, {nbytes} needed")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _qkv_shape(p: Params):
    return (p.B, p.H, p.L_src + p.L_ctx, p.D)


def _check_qkv(p: Params, *ts, names="QKV"):
    torch = _torch()
    shape = _qkv_shape(p)
    dev = ts[0].device if ts and isinstance(ts[0], torch.Tensor) else None
    for name, t in zip(names if len(names) == len(ts) else [f"tensor {k}" for k in range(len(ts))], ts):
        _req(name, t, shape, torch.bfloat16, dev)
    return dev


def _nz(t) -> int | None:
    return t.data_ptr() if t.numel() else None


def _empty(shape, dtype, device):
    return _torch().empty(shape, dtype=dtype, device=device)


def forward(Q, K, V, p: Params, debug: bool = False, out=None, workspace=None):
    """ISA forward (steps 1-6). Returns O, or (O, debug dict) when debug=True.
    `out` (bf16, Q's shape) and `workspace` (at least plan()["workspace_bytes"]
    bytes) may be given to avoid allocation."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    pl = plan(p)
    if out is not None:
        _req("out", out, _qkv_shape(p), torch.bfloat16, dev)
    O = out if out is not None else torch.empty_like(Q)
    if workspace is not None:
        _req_bytes("workspace", workspace, pl["workspace_bytes"], dev)
    ws = workspace if workspace is not None else _empty((pl["workspace_bytes"],), torch.uint8, dev)
    dbg_t, dbg_c = None, None
    if debug:
        dbg_t = {
            "qc": _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev),
            "kc": _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev),
            "ctx_score": _empty((p.B, p.H, pl["N_ctx"]), torch.float64, dev),
            "ctx_idx": _empty((p.B, p.H, pl["k_ctx"]), torch.int32, dev),
            "sharpness": _empty((p.B, p.H, pl["N"]), torch.float64, dev),
            "sharp_idx": _empty((p.B, p.H, pl["n_sharp"]), torch.int32, dev),
            "flat_idx": _empty((p.B, p.H, pl["n_flat"]), torch.int32, dev),
            "flat_exact_idx": _empty((p.B, p.H, pl["n_flat"], pl["k_ns"]), torch.int32, dev),
        }
        dbg_c = IsaDebug(**{k: v.data_ptr() for k, v in dbg_t.items()})
    rc = lib().isa_forward(ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                           O.data_ptr(), ws.data_ptr(), _nbytes(ws),
                           ctypes.byref(dbg_c) if dbg_c is not None else None, _stream(dev))
    _check("isa_forward", rc)
    return (O, dbg_t) if debug else O


def forward_noalloc(Q, K, V, p: Params, out=None):
    """isa_forward_noalloc: the forward with the library's static device
    scratch as its workspace (nothing allocated by the library; `out` may be
    given so that nothing is allocated here either). Raises IsaError with
    ISA_ERR_SCRATCH when plan()["noalloc_bytes"] exceeds the scratch size."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    if out is not None:
        _req("out", out, _qkv_shape(p), torch.bfloat16, dev)
    O = out if out is not None else torch.empty_like(Q)
    _check("isa_forward_noalloc", lib().isa_forward_noalloc(
        ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), None, _stream(dev)))
    return O


def init():
    """isa_init: one-time set-up of the current device (optional)."""
    _check("isa_init", lib().isa_init())


def workspace(p: Params, device):
    """A workspace for forward() and backward() (plan()["workspace_bytes"] bytes)."""
    torch = _torch()
    return _empty((plan(p)["workspace_bytes"],), torch.uint8, device)


def backward(Q, K, V, O, dO, p: Params, workspace, out=None):
    """Gradients (dQ, dK, dV) of sum(dO * O), selections held fixed. Q, K, V, O
    and `workspace` must be those of the forward() call that produced O (its
    workspace argument, unmodified since). `out` = (dQ, dK, dV) buffers, or
    None to allocate them."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V, O, dO, names=("Q", "K", "V", "O", "dO"))
    _req_bytes("workspace", workspace, plan(p)["workspace_bytes"], dev)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a (dQ, dK, dV) triple")
        for name, t in zip(("dQ", "dK", "dV"), out):
            _req(name, t, _qkv_shape(p), torch.bfloat16, dev)
    dQ, dK, dV = out if out is not None else (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    _check("isa_backward", lib().isa_backward(
        ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dO.data_ptr(),
        dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), workspace.data_ptr(), _nbytes(workspace),
        _stream(dev)))
    return dQ, dK, dV


def pool_coarse(Q, K, V, p: Params):
    """Step (1) pooling: returns (qc, kc fp64, kc_bf16, vc_bf16)."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    pl = plan(p)
    qc = _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev)
    kc = _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev)
    kcb = _empty((p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    vcb = _empty((p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    _check("isa_pool_coarse", lib().isa_pool_coarse(ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(),
                                                    V.data_ptr(), qc.data_ptr(), kc.data_ptr(),
                                                    kcb.data_ptr(), vcb.data_ptr(), _stream(dev)))
    return qc, kc, kcb, vcb


def rope_pool_coarse(Q, K, V, p: Params):
    """Decoupled RoPE fused with step (1): returns (Qr, Kr, qc, kc, kc_bf16, vc_bf16)."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    pl = plan(p)
    Qr = _empty(tuple(Q.shape), torch.bfloat16, dev)
    Kr = _empty(tuple(K.shape), torch.bfloat16, dev)
    qc = _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev)
    kc = _empty((p.B, p.H, pl["N"], p.D), torch.float64, dev)
    kcb = _empty((p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    vcb = _empty((p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    ws = _empty((max(pl["rope_bytes"], 1),), torch.uint8, dev)
    _check("isa_rope_pool_coarse", lib().isa_rope_pool_coarse(
        ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(), V.data_ptr(), Qr.data_ptr(),
        Kr.data_ptr(), qc.data_ptr(), kc.data_ptr(), kcb.data_ptr(), vcb.data_ptr(),
        ws.data_ptr(), _nbytes(ws), _stream(dev)))
    return Qr, Kr, qc, kc, kcb, vcb


def _check_coarse(p: Params, pl: dict, qc, kc):
    torch = _torch()
    shape = (p.B, p.H, pl["N"], p.D)
    _req("qc", qc, shape, torch.float64)
    _req("kc", kc, shape, torch.float64, qc.device)
    return qc.device


def _check_ctx(p: Params, pl: dict, ctx_idx, dev):
    _req("ctx_idx", ctx_idx, (p.B, p.H, pl["k_ctx"]), _torch().int32, dev)


def ctx_topk(qc, kc, p: Params):
    """Step (2): returns (ctx_idx int32 global ids, ctx_score fp64)."""
    torch = _torch()
    pl = plan(p)
    dev = _check_coarse(p, pl, qc, kc)
    idx = _empty((p.B, p.H, pl["k_ctx"]), torch.int32, dev)
    score = _empty((p.B, p.H, pl["N_ctx"]), torch.float64, dev)
    _check("isa_ctx_topk", lib().isa_ctx_topk(ctypes.byref(p.c()), qc.data_ptr(), kc.data_ptr(),
                                              _nz(idx), _nz(score), _stream(dev)))
    return idx, score


def sharpness_split(qc, kc, ctx_idx, p: Params):
    """Steps (1) coarse rows, (3), (5) selection: returns
    (sharpness, sharp_idx, flat_idx, flat_exact_idx)."""
    torch = _torch()
    pl = plan(p)
    dev = _check_coarse(p, pl, qc, kc)
    _check_ctx(p, pl, ctx_idx, dev)
    sharp = _empty((p.B, p.H, pl["N"]), torch.float64, dev)
    si = _empty((p.B, p.H, pl["n_sharp"]), torch.int32, dev)
    fi = _empty((p.B, p.H, pl["n_flat"]), torch.int32, dev)
    ei = _empty((p.B, p.H, pl["n_flat"], pl["k_ns"]), torch.int32, dev)
    ws = _empty((pl["scores_bytes"],), torch.uint8, dev)
    _check("isa_sharpness_split", lib().isa_sharpness_split(
        ctypes.byref(p.c()), qc.data_ptr(), kc.data_ptr(), _nz(ctx_idx), sharp.data_ptr(),
        _nz(si), _nz(fi), _nz(ei), ws.data_ptr(), _nbytes(ws), _stream(dev)))
    return sharp, si, fi, ei


def sharp_attn(Q, K, V, ctx_idx, sharp_idx, p: Params, out=None):
    """Step (4): writes the sharp rows of `out` (allocated zero if None)."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    pl = plan(p)
    _check_ctx(p, pl, ctx_idx, dev)
    _req("sharp_idx", sharp_idx, (p.B, p.H, pl["n_sharp"]), torch.int32, dev)
    if out is not None:
        _req("out", out, _qkv_shape(p), torch.bfloat16, dev)
    O = out if out is not None else torch.zeros_like(Q)
    _check("isa_sharp_attn", lib().isa_sharp_attn(ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(),
                                                  V.data_ptr(), _nz(ctx_idx), _nz(sharp_idx),
                                                  O.data_ptr(), _stream(dev)))
    return O


def flat_taylor_attn(Q, K, V, kc_bf16, vc_bf16, ctx_idx, flat_idx, flat_exact_idx, p: Params,
                     out=None):
    """Step (5): writes the flat rows of `out` (allocated zero if None)."""
    torch = _torch()
    dev = _check_qkv(p, Q, K, V)
    pl = plan(p)
    _req("kc_bf16", kc_bf16, (p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    _req("vc_bf16", vc_bf16, (p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    _check_ctx(p, pl, ctx_idx, dev)
    _req("flat_idx", flat_idx, (p.B, p.H, pl["n_flat"]), torch.int32, dev)
    _req("flat_exact_idx", flat_exact_idx, (p.B, p.H, pl["n_flat"], pl["k_ns"]), torch.int32, dev)
    if out is not None:
        _req("out", out, _qkv_shape(p), torch.bfloat16, dev)
    O = out if out is not None else torch.zeros_like(Q)
    _check("isa_flat_taylor_attn", lib().isa_flat_taylor_attn(
        ctypes.byref(p.c()), Q.data_ptr(), K.data_ptr(), V.data_ptr(), kc_bf16.data_ptr(),
        vc_bf16.data_ptr(), _nz(ctx_idx), _nz(flat_idx), _nz(flat_exact_idx), O.data_ptr(),
        _stream(dev)))
    return O


def coarse_residual(qc, kc, vc_bf16, ctx_idx, O, p: Params):
    """Step (6): adds gamma * O_coarse to every token row of O in place."""
    torch = _torch()
    pl = plan(p)
    dev = _check_coarse(p, pl, qc, kc)
    _req("vc_bf16", vc_bf16, (p.B, p.H, pl["N"], p.D), torch.bfloat16, dev)
    _check_ctx(p, pl, ctx_idx, dev)
    _req("O", O, _qkv_shape(p), torch.bfloat16, dev)
    ws = _empty((pl["scores_bytes"],), torch.uint8, dev)
    _check("isa_coarse_residual", lib().isa_coarse_residual(
        ctypes.byref(p.c()), qc.data_ptr(), kc.data_ptr(), vc_bf16.data_ptr(), _nz(ctx_idx),
        O.data_ptr(), ws.data_ptr(), _nbytes(ws), _stream(dev)))
    return O


def dense_attn(Q, K, V, out=None):
    """Dense softmax attention baseline over all tokens, [B,H,L,D] bf16."""
    torch = _torch()
    if not isinstance(Q, torch.Tensor) or Q.dim() != 4:
        raise ValueError("Q must be a [B, H, L, D] tensor")
    B, H, L, D = Q.shape
    for name, t in zip("QKV", (Q, K, V)):
        _req(name, t, Q.shape, torch.bfloat16, Q.device)
    if out is not None:
        _req("out", out, Q.shape, torch.bfloat16, Q.device)
    O = out if out is not None else torch.empty_like(Q)
    _check("isa_dense_attn", lib().isa_dense_attn(B, H, L, D, Q.data_ptr(), K.data_ptr(),
                                                  V.data_ptr(), O.data_ptr(), _stream(Q.device)))
    return O
