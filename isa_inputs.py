"""Seeded synthetic inputs for In-context Sparse Attention (ISA).

This module is shared by the CPU oracle, the tests and the benchmark. It
contains only the input recipe (clustered Q/K, random V, bf16 rounding). None
of the method's arithmetic lives here.

The pages describe in-context video editing with two token segments
concatenated into one attention sequence, source first, then context
(rainbus.top summary of arXiv 2605.04569, section "Prerequisites",
in-context learning paragraph). They benchmark attention only on synthetic
latency sweeps, so there is no public dataset to stand in for. The recipe
below imitates the structure the method relies on:

* query/key tokens grouped into clusters, with a fixed cluster id per
  64-token generator block, so coarse block scores are informative;
* context keys scaled by 0.5, modelling the observation that context tokens
  are less salient than source tokens (same page, "Motivation", Fig. 5);
* query blocks drawn at temperature 1 or 4, so that sharp and flat coarse
  softmax rows both occur (same page, "Core method": the query split by
  sharpness).

Generator blocks are always 64 tokens and segment-aligned, independent of the
method's block size b, so a sweep over b sees identical inputs.
"""
from __future__ import annotations

import numpy as np

N_CENTRES = 16
GEN_BLOCK = 64
WITHIN_STD = 0.3
CTX_K_SCALE = 0.5
TEMPERATURES = (1.0, 4.0)


def round_to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 to bf16 with round-to-nearest-even.

    Returns (bits uint16, value as float32). NaN/Inf are not produced by the
    generator and are not handled specially.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    val = (r.astype(np.uint32) << 16).view(np.float32)
    return r, val


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _segment_blocks(L_src: int, L_ctx: int, g: int):
    out = []
    for seg_start, seg_len in ((0, L_src), (L_src, L_ctx)):
        for s in range(0, seg_len, g):
            out.append((seg_start + s, min(g, seg_len - s)))
    return out


def make_head(stream: int, b_idx: int, h: int, L_src: int, L_ctx: int, D: int):
    """Generate fp32 (Q, K, V) of shape [L, D] for one (batch, head).

    Stream: numpy default_rng([stream, b_idx, h]) (`stream` is the
    workload's seed stream, WORKLOADS[name]["stream"]); each head can be
    regenerated on its own.
    """
    rng = np.random.default_rng([stream, b_idx, h])
    L = L_src + L_ctx
    centres = rng.standard_normal((N_CENTRES, D)).astype(np.float32)
    blocks = _segment_blocks(L_src, L_ctx, GEN_BLOCK)
    z = rng.integers(0, N_CENTRES, size=len(blocks))
    tau = np.asarray(TEMPERATURES, dtype=np.float32)[rng.integers(0, 2, size=len(blocks))]
    eq = rng.standard_normal((L, D)).astype(np.float32) * np.float32(WITHIN_STD)
    ek = rng.standard_normal((L, D)).astype(np.float32) * np.float32(WITHIN_STD)
    V = rng.standard_normal((L, D)).astype(np.float32)
    tok_centre = np.empty(L, dtype=np.int64)
    tok_tau = np.empty(L, dtype=np.float32)
    for gi, (s, n) in enumerate(blocks):
        tok_centre[s:s + n] = z[gi]
        tok_tau[s:s + n] = tau[gi]
    C = centres[tok_centre]
    Q = (C + eq) / tok_tau[:, None]
    K = C + ek
    K[L_src:] *= np.float32(CTX_K_SCALE)
    return Q.astype(np.float32), K.astype(np.float32), V


def make_inputs(stream: int, B: int, H: int, L_src: int, L_ctx: int, D: int,
                heads=None, bf16: bool = True):
    """Generate Q, K, V as [B, H, L, D] arrays.

    With bf16=True returns (bits uint16, values float32) per tensor, i.e. a
    dict {"Q": (bits, f32), ...}; otherwise float32 arrays. `heads` restricts
    generation to a list of (b_idx, h) pairs (others left zero).
    """
    L = L_src + L_ctx
    sel = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    out = {}
    names = ("Q", "K", "V")
    if bf16:
        for nm in names:
            out[nm] = (np.zeros((B, H, L, D), np.uint16), np.zeros((B, H, L, D), np.float32))
    else:
        for nm in names:
            out[nm] = np.zeros((B, H, L, D), np.float32)
    for (b, h) in sel:
        qkv = make_head(stream, b, h, L_src, L_ctx, D)
        for nm, x in zip(names, qkv):
            if bf16:
                bits, val = round_to_bf16(x)
                out[nm][0][b, h] = bits
                out[nm][1][b, h] = val
            else:
                out[nm][b, h] = x
    return out


# Workload shapes (B, H, D, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns) and
# the seed stream each one's inputs are drawn from.
DEFAULT_RATIOS = dict(alpha_s=0.125, alpha_f=0.5, alpha_ns=0.0625)
WORKLOADS = {
    "tiny": dict(stream=1, B=1, H=2, D=64, L_src=1024, L_ctx=1024, b=64, **DEFAULT_RATIOS),
    "16k": dict(stream=2, B=1, H=40, D=128, L_src=8192, L_ctx=8192, b=64, **DEFAULT_RATIOS),
    "23768_ragged": dict(stream=3, B=1, H=40, D=128, L_src=11884, L_ctx=11884, b=64, **DEFAULT_RATIOS),
    "64k": dict(stream=4, B=1, H=40, D=128, L_src=32768, L_ctx=32768, b=64, **DEFAULT_RATIOS),
    "128k": dict(stream=5, B=1, H=40, D=128, L_src=65536, L_ctx=65536, b=64, **DEFAULT_RATIOS),
}
