"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every entry point declared in include/isa.h, isa_plan agrees with the oracle's
counts, and invalid calls fail with the documented codes before anything is
launched."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def isa():
    import block_sparse_attention_blockwise_amd as isa
    if not os.path.exists(isa.LIB_PATH):
        from block_sparse_attention_blockwise_amd import _build
        _build.build()
    isa.lib()
    return isa


def _declared():
    txt = open(os.path.join(ROOT, "include", "isa.h")).read()
    return re.findall(r"ISA_API\s+[\w\s\*]+?\b(isa_\w+)\s*\(", txt)


def test_exports_every_declared_symbol(isa):
    names = _declared()
    assert set(names) == set(isa.EXPORTED)
    nm = subprocess.run(["nm", "-D", "--defined-only", isa.LIB_PATH], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in nm.stdout.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
        assert getattr(isa.lib(), n) is not None


def test_binding_declares_every_signature(isa):
    """Every entry point has its argument types declared in the binding (an
    undeclared one would pass pointers as C ints), matching the header's
    parameter count."""
    txt = open(os.path.join(ROOT, "include", "isa.h")).read()
    for name, args in re.findall(r"ISA_API\s+[\w\s\*]+?\b(isa_\w+)\s*\(([^)]*)\)", txt):
        fn = getattr(isa.lib(), name)
        assert fn.argtypes is not None, name
        params = [a for a in args.split(",") if a.strip() and a.strip() != "void"]
        assert len(fn.argtypes) == len(params), name


def test_plan_matches_oracle_counts(isa):
    from oracle import isa_oracle
    import isa_inputs
    cases = []
    for c in isa_inputs.WORKLOADS.values():
        cases.append((c["L_src"], c["L_ctx"], c["D"], c["b"], c["alpha_s"], c["alpha_f"], c["alpha_ns"]))
    for b in (32, 64):
        for a_s in (0.125, 0.25):
            for a_ns in (0.0625, 0.125):
                for a_f in (0.25, 0.5, 0.75):
                    cases.append((65536, 65536, 128, b, a_s, a_f, a_ns))
    cases += [(1, 0, 64, 32, 0.5, 0.5, 0.5), (100, 0, 64, 32, 0.125, 0.5, 0.0625),
              (11884, 11884, 128, 64, 0.1, 0.3, 0.07), (777, 333, 64, 64, 1.0, 1.0, 1.0),
              (777, 333, 64, 64, 0.0, 0.0, 0.0)]
    for (Ls, Lc, D, b, a_s, a_f, a_ns) in cases:
        pl = isa.plan(isa.Params(1, 40, Ls, Lc, D, b, a_s, a_f, a_ns))
        o = isa_oracle.make_plan(Ls, Lc, b, a_s, a_f, a_ns)
        for k in ("N_src", "N_ctx", "N", "k_ctx", "N_kv", "n_flat", "n_sharp", "k_ns"):
            assert pl[k] == getattr(o, k), (k, Ls, Lc, b, a_s, a_f, a_ns)
        # the coarse scores are never stored: no N * N_kv term without the
        # residual; only the exact-set kernel's row scratch (256 slots of 16
        # rows of J, fp64) when 16 rows of J (N_kv > 640) do not fit LDS
        ftk = 256 * 16 * o.N_kv * 8 if (o.N_kv > 640 and o.n_flat > 0 and o.k_ns > 0) else 0
        assert pl["scores_bytes"] == (40 * o.N * 8 + 255) // 256 * 256 + (ftk + 255) // 256 * 256
        assert pl["rope_bytes"] == 0
        # only the gamma residual keeps the coarse rows S[i, J] (fp64)
        pg = isa.plan(isa.Params(1, 40, Ls, Lc, D, b, a_s, a_f, a_ns, gamma=0.5))
        assert pg["scores_bytes"] >= 40 * o.N * o.N_kv * 8
        assert pg["workspace_bytes"] - pl["workspace_bytes"] >= 40 * o.N * o.N_kv * 8


def test_plan_rope_workspace(isa):
    """RoPE adds the rotated Q and K and the cos/sin table to the forward
    workspace; the table covers max(L_src, L_ctx) positions."""
    for (Ls, Lc, D) in ((1024, 1024, 64), (777, 333, 128), (100, 0, 64), (333, 777, 128)):
        off = isa.plan(isa.Params(2, 3, Ls, Lc, D, 64))
        on = isa.plan(isa.Params(2, 3, Ls, Lc, D, 64, rope_base=10000.0))
        assert on["rope_bytes"] >= max(Ls, Lc) * (D // 2) * 8
        assert on["workspace_bytes"] >= off["workspace_bytes"] + 2 * 6 * (Ls + Lc) * D * 2 + on["rope_bytes"]


def _params(isa, **kw):
    base = dict(B=1, H=2, L_src=1024, L_ctx=1024, D=128, b=64, alpha_s=0.125, alpha_f=0.5,
                alpha_ns=0.0625, gamma=0.0, rope_base=0.0)
    base.update(kw)
    return isa.IsaParams(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(L_src=0), -1), (dict(L_ctx=-1), -1), (dict(B=0), -1), (dict(H=0), -1),
    (dict(D=0), -1), (dict(b=0), -1),
    (dict(alpha_s=float("nan")), -1), (dict(alpha_f=1.5), -1), (dict(alpha_ns=-0.1), -1),
    (dict(gamma=float("nan")), -1), (dict(gamma=float("inf")), -1), (dict(gamma=1e300), -1),
    (dict(rope_base=float("nan")), -1), (dict(rope_base=float("inf")), -1),
    (dict(rope_base=-10000.0), -1), (dict(rope_base=1.0), -1), (dict(rope_base=0.5), -1),
    (dict(D=96), -2), (dict(D=256), -2), (dict(b=16), -2), (dict(b=128), -2),
    (dict(L_src=64 * 4097), -2), (dict(L_ctx=64 * 4097), -2),
    (dict(L_src=64 * 4000, L_ctx=64 * 4000, alpha_s=0.05), -2),   # N_kv > 4096
    (dict(B=256, H=256), -2),                                       # B*H > 65535
])
def test_plan_rejects(isa, kw, code):
    out = isa.IsaPlan()
    assert isa.lib().isa_plan(ctypes.byref(_params(isa, **kw)), ctypes.byref(out)) == code


def test_calls_fail_before_launch(isa):
    L = isa.lib()
    p = _params(isa)
    fake = 0x1000   # never dereferenced: every call below fails validation first
    assert L.isa_plan(None, None) == -1
    assert L.isa_forward(None, fake, fake, fake, fake, fake, 1 << 40, None, None) == -1
    assert L.isa_forward(ctypes.byref(p), None, fake, fake, fake, fake, 1 << 40, None, None) == -1
    assert L.isa_forward(ctypes.byref(p), fake, fake, fake, fake, fake, 16, None, None) == -3
    assert L.isa_sharpness_split(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                                 16, None) == -3
    assert L.isa_sharpness_split(ctypes.byref(p), fake, fake, None, fake, fake, fake, fake, fake,
                                 1 << 40, None) == -1
    assert L.isa_pool_coarse(ctypes.byref(p), fake, None, fake, fake, fake, None, None, None) == -1
    assert L.isa_ctx_topk(ctypes.byref(p), fake, fake, None, None, None) == -1
    assert L.isa_sharp_attn(ctypes.byref(p), fake, fake, fake, None, fake, fake, None) == -1
    assert L.isa_flat_taylor_attn(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake,
                                  fake, fake, None) == -1
    assert L.isa_coarse_residual(ctypes.byref(p), fake, fake, fake, fake, None, fake, 1 << 40, None) == -1
    assert L.isa_coarse_residual(ctypes.byref(_params(isa, gamma=0.5)), fake, fake, fake, fake, fake, fake,
                                 16, None) == -3
    rp = _params(isa, rope_base=10000.0)
    assert L.isa_rope_pool_coarse(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                                  fake, fake, 1 << 40, None) == -1      # RoPE off
    assert L.isa_rope_pool_coarse(ctypes.byref(rp), fake, fake, fake, None, fake, fake, fake, fake,
                                  fake, fake, 1 << 40, None) == -1
    assert L.isa_rope_pool_coarse(ctypes.byref(rp), fake, fake, fake, fake, fake, fake, fake, fake,
                                  fake, fake, 16, None) == -3
    assert L.isa_backward(ctypes.byref(p), fake, fake, fake, fake, None, fake, fake, fake, fake,
                          1 << 40, None) == -1
    assert L.isa_backward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                          16, None) == -3
    g = _params(isa, gamma=float("nan"))
    assert L.isa_backward(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                          1 << 40, None) == -1
    # the residual's scratch makes the workspace larger
    pl0, pl1 = isa.IsaPlan(), isa.IsaPlan()
    assert L.isa_plan(ctypes.byref(p), ctypes.byref(pl0)) == 0
    assert L.isa_plan(ctypes.byref(_params(isa, gamma=0.5)), ctypes.byref(pl1)) == 0
    assert pl1.workspace_bytes > pl0.workspace_bytes
    assert L.isa_dense_attn(1, 1, 0, 128, fake, fake, fake, fake, None) == -1
    assert L.isa_dense_attn(1, 1, 16, 96, fake, fake, fake, fake, None) == -2
    assert L.isa_dense_attn(256, 256, 16, 64, fake, fake, fake, fake, None) == -2
    # a head's rows beyond 32-bit byte offsets
    assert L.isa_dense_attn(1, 1, 1 << 23, 128, fake, fake, fake, fake, None) == -2
    assert L.isa_dense_attn(1, 1, 16, 128, None, fake, fake, fake, None) == -1
    # 16-byte alignment of the vector-accessed tensors
    odd = fake + 8
    assert L.isa_forward(ctypes.byref(p), odd, fake, fake, fake, fake, 1 << 40, None, None) == -1
    assert L.isa_backward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, odd, fake, fake,
                          1 << 40, None) == -1
    assert L.isa_sharp_attn(ctypes.byref(p), fake, fake, fake, fake, fake, odd, None) == -1
    assert L.isa_dense_attn(1, 1, 16, 128, fake, odd, fake, fake, None) == -1
    assert L.isa_pool_coarse(ctypes.byref(p), fake, fake, odd, fake, fake, None, None, None) == -1
    assert L.isa_pool_coarse(ctypes.byref(p), fake, fake, fake, odd, fake, None, None, None) == -1
    assert L.isa_pool_coarse(ctypes.byref(p), fake, fake, fake, fake, fake, None, odd, None) == -1
    assert L.isa_ctx_topk(ctypes.byref(p), fake, odd, fake, None, None) == -1
    assert L.isa_sharpness_split(ctypes.byref(p), odd, fake, fake, fake, fake, fake, fake, fake,
                                 1 << 40, None) == -1
    assert L.isa_sharpness_split(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, odd,
                                 1 << 40, None) == -1
    assert L.isa_coarse_residual(ctypes.byref(p), fake, fake, fake, fake, odd, fake, 1 << 40, None) == -1
    assert L.isa_coarse_residual(ctypes.byref(p), fake, fake, odd, fake, fake, fake, 1 << 40, None) == -1
    bad = _params(isa, D=96)
    assert L.isa_forward(ctypes.byref(bad), fake, fake, fake, fake, fake, 1 << 40, None, None) == -2
    # the allocation-free forward: arguments first, then the static scratch size
    assert L.isa_forward_noalloc(ctypes.byref(p), fake, None, fake, fake, None, None) == -1
    assert L.isa_forward_noalloc(ctypes.byref(p), fake, fake, odd, fake, None, None) == -1
    assert L.isa_forward_noalloc(ctypes.byref(bad), fake, fake, fake, fake, None, None) == -2


def test_noalloc_scratch_limit(isa):
    """isa_plan reports the scratch the allocation-free forward needs (the
    forward's own buffers, no backward state); requests beyond
    ISA_NOALLOC_SCRATCH_BYTES are refused with ISA_ERR_SCRATCH before any
    HIP call."""
    L = isa.lib()
    fake = 0x1000
    hdr = open(os.path.join(ROOT, "include", "isa.h")).read()
    m = re.search(r"#define ISA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == isa.NOALLOC_SCRATCH_BYTES
    small = isa.plan(isa.Params(1, 40, 8192, 8192, 128, 64))          # 16384 tokens fit
    assert small["noalloc_bytes"] <= isa.NOALLOC_SCRATCH_BYTES
    assert small["noalloc_bytes"] < small["workspace_bytes"]
    big = _params(isa, B=1, H=40, L_src=32768, L_ctx=32768)          # 65536 tokens do not
    pl = isa.IsaPlan()
    assert L.isa_plan(ctypes.byref(big), ctypes.byref(pl)) == 0
    assert pl.noalloc_bytes > isa.NOALLOC_SCRATCH_BYTES
    assert L.isa_forward_noalloc(ctypes.byref(big), fake, fake, fake, fake, None, None) == isa.ISA_ERR_SCRATCH
    assert "scratch" in isa.strerror(isa.ISA_ERR_SCRATCH)


def test_init_without_device(isa):
    """isa_init sets up the current device; on a host without a usable HIP
    device it reports ISA_ERR_HIP instead of failing in another way."""
    torch = pytest.importorskip("torch")
    rc = isa.lib().isa_init()
    if torch.cuda.device_count() == 0:
        assert rc == isa.ISA_ERR_HIP
    else:
        assert rc == isa.ISA_OK


def test_strerror(isa):
    for code in (0, -1, -2, -3, -4, -5, 7):
        s = isa.strerror(code)
        assert isinstance(s, str) and s
    assert "workspace" in isa.strerror(-3)


def test_binding_refuses_host_tensors(isa):
    """The binding checks every tensor before any library call: host
    tensors, non-tensors and wrong shapes are refused with an exception."""
    torch = pytest.importorskip("torch")
    p = isa.Params(1, 2, 128, 64, 64, 64)
    x = torch.zeros(1, 2, 192, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        isa.forward(x, x, x, p)
    with pytest.raises(ValueError, match="HIP device"):
        isa.dense_attn(x, x, x)
    with pytest.raises(TypeError, match="torch.Tensor"):
        isa.forward(x.float().numpy(), x, x, p)
    with pytest.raises(ValueError, match="HIP device"):
        isa.ctx_topk(torch.zeros(1, 2, 4, 64, dtype=torch.float64),
                     torch.zeros(1, 2, 4, 64, dtype=torch.float64), p)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import block_sparse_attention_blockwise_amd as isa
    monkeypatch.setattr(isa, "_lib", None)
    monkeypatch.setattr(isa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        isa.lib()


def test_header_is_plain_c_and_links(isa, tmp_path):
    """include/isa.h compiles as C99 on its own, and a C program linked
    against the library can plan a forward pass and read status strings (no
    GPU needed)."""
    src = tmp_path / "client.c"
    src.write_text(r'''
#include <stdio.h>
#include "isa.h"
int main(void) {
  isa_params_t p = {1, 40, 32768, 32768, 128, 64, 0.125, 0.5, 0.0625, 0.0, 0.0};
  isa_plan_t pl;
  int rc = isa_plan(&p, &pl);
  if (rc != ISA_OK) { printf("plan failed: %s\n", isa_strerror(rc)); return 1; }
  printf("%d %d %d %d %d %d %zu\n", pl.N, pl.k_ctx, pl.N_kv, pl.n_flat, pl.n_sharp, pl.k_ns,
         pl.workspace_bytes);
  p.D = 96;
  return isa_plan(&p, &pl) == ISA_ERR_UNSUPPORTED ? 0 : 2;
}
''')
    exe = tmp_path / "client"
    lib_dir = os.path.dirname(isa.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-L", lib_dir, "-lisa_mi355x", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    N, k_ctx, N_kv, n_flat, n_sharp, k_ns, ws = (int(x) for x in r.stdout.split())
    assert (N, k_ctx, N_kv, n_flat, n_sharp, k_ns) == (1024, 64, 576, 512, 512, 36)
    assert ws > 0
