"""GPU parity of the ISA backward pass (isa_backward through the C ABI)
against the oracle's fp64 gradients with the selections held fixed.

Tolerance, from the arithmetic: the kernels round the probabilities and the
score gradients dS to bf16 before the matrix-core products (relative error
2^-9 each), accumulate in fp32, and round the gradients to bf16 (2^-9); the
forward's Taylor operands Kc, Vc are bf16 while the oracle's are fp64. Each
gradient element is a sum of many such terms with cancellation (the rows of
dS sum to zero), so the bound is taken relative to the tensor's RMS: the
rounding errors add like a random walk, ||gpu - oracle|| <= 0.02 * ||oracle||
(about ten times the per-term 2^-9), and the largest single deviation, a
several-sigma tail over ~10^5 elements, max |gpu - oracle| <= 0.3 * rms(oracle)."""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import isa_inputs
from oracle import isa_oracle
from parity_util import bf16_tensor

STREAM = {name: w["stream"] for name, w in isa_inputs.WORKLOADS.items()}

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
isa = pytest.importorskip("block_sparse_attention_blockwise_amd")

MAX_RMS = 0.3
REL_L2 = 0.02


def log(msg):
    print(f"[gpu-bwd {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    isa.lib()
    return torch.device("cuda:0")


def _dO(p, seed):
    """Seeded output gradient ~N(0, 1), rounded to bf16 (bits, values)."""
    rng = np.random.default_rng([99, seed])
    x = rng.standard_normal((p.B, p.H, p.L_src + p.L_ctx, p.D)).astype(np.float32)
    return isa_inputs.round_to_bf16(x)


def _run(p, inp, dO_bits, dev):
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    dO = bf16_tensor(dO_bits, dev)
    ws = isa.workspace(p, dev)
    O, dbg = isa.forward(Q, K, V, p, debug=True, workspace=ws)
    dQ, dK, dV = isa.backward(Q, K, V, O, dO, p, ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    return dict(dQ=f(dQ), dK=f(dK), dV=f(dV), O=f(O),
                sel={k: v.cpu().numpy() for k, v in dbg.items()})


def _compare(name, got, ref):
    err = np.abs(got - ref)
    rms = float(np.sqrt((ref ** 2).mean()))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert np.isfinite(got).all(), f"{name}: non-finite"
    log(f"  {name}: max-abs {err.max():.3e} (rms {rms:.3e}, ratio {err.max() / max(rms, 1e-30):.3f}) rel-L2 {rel:.2e}")
    assert err.max() <= MAX_RMS * rms and rel <= REL_L2, (name, float(err.max()), rms, rel)
    return rel


def _oracle_grads(plan, inp, dO_vals, bi, h, sel, gamma=0.0, rope_base=0.0):
    Qv, Kv, Vv = (inp[n][1][bi, h] for n in "QKV")
    if rope_base:
        Qv = isa_oracle.rope(Qv, plan.L_src, plan.L_ctx, rope_base)
        Kv = isa_oracle.rope(Kv, plan.L_src, plan.L_ctx, rope_base)
    selections = dict(ctx_idx=np.asarray(sel["ctx_idx"][bi, h], dtype=np.int64) - plan.N_src,
                      sharp_idx=sel["sharp_idx"][bi, h], flat_idx=sel["flat_idx"][bi, h],
                      flat_exact_idx=sel["flat_exact_idx"][bi, h])
    ref_sel = isa_oracle.isa_head(Qv, Kv, Vv, plan, compute_output=False)
    assert np.array_equal(ref_sel.ctx_idx, selections["ctx_idx"])
    assert np.array_equal(ref_sel.sharp_idx, selections["sharp_idx"])
    assert np.array_equal(ref_sel.flat_exact_idx, selections["flat_exact_idx"].reshape(ref_sel.flat_exact_idx.shape))
    gq, gk, gv = isa_oracle.isa_head_backward(Qv, Kv, Vv, dO_vals[bi, h], plan, gamma=gamma)
    if rope_base:
        gq = isa_oracle.rope_backward(gq, plan.L_src, plan.L_ctx, rope_base)
        gk = isa_oracle.rope_backward(gk, plan.L_src, plan.L_ctx, rope_base)
    return gq, gk, gv


def _check_all_rows(p, stream=1, seed=0, heads=None):
    inp = isa_inputs.make_inputs(stream, p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, seed)
    res = _run(p, inp, dO_bits, torch.device("cuda:0"))
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for (bi, h) in (heads or [(x, y) for x in range(p.B) for y in range(p.H)]):
        log(f"head ({bi},{h})")
        gq, gk, gv = _oracle_grads(plan, inp, dO_vals, bi, h, res["sel"], gamma=p.gamma,
                                   rope_base=p.rope_base)
        _compare("dQ", res["dQ"][bi, h], gq)
        _compare("dK", res["dK"][bi, h], gk)
        _compare("dV", res["dV"][bi, h], gv)
    return res, plan


@pytest.mark.parametrize("D,b", [(128, 64), (64, 32), (128, 32), (64, 64)])
def test_backward_small_all_rows(dev, D, b):
    """Ragged segments (700 + 451 tokens), sharp and flat blocks, pruned
    context blocks; every gradient element against the oracle."""
    p = isa.Params(1, 2, 700, 451, D, b, 0.25, 0.5, 0.125)
    _check_all_rows(p)


def test_backward_batch_and_heads(dev):
    p = isa.Params(2, 3, 333, 290, 128, 64, 0.5, 0.5, 0.25)
    _check_all_rows(p, heads=[(0, 0), (1, 2)])


def test_backward_ordered_grids(dev):
    """The dK/dV grid takes each head's key chunks longest stream first and
    the flat dQ grid the forward's flat-block order, each XCD taking a
    contiguous run when the workgroup count is a multiple of 8: B*H = 8
    distinct heads, b = 64, many flat blocks per kept block; every gradient
    element of every head against the oracle."""
    p = isa.Params(2, 4, 1536, 1600, 128, 64, 0.25, 0.75, 0.25)
    pl = isa.plan(p)
    assert (pl["n_flat"] * p.B * p.H) % 8 == 0 and pl["k_ns"] > 1
    _check_all_rows(p)


@pytest.mark.parametrize("a_s,a_f,a_ns,L_ctx", [
    (1.0, 0.0, 0.25, 451),    # dense special case: every block sharp over every token
    (1.0, 1.0, 0.0, 451),     # pure Taylor: every block flat over pooled keys only
    (0.25, 1.0, 1.0, 451),    # alpha_ns = 1: flat blocks exact over J, no pooled keys
    (0.125, 0.5, 0.125, 0),   # no context segment
])
def test_backward_special_cases(dev, a_s, a_f, a_ns, L_ctx):
    p = isa.Params(1, 2, 700, L_ctx, 128, 64, a_s, a_f, a_ns)
    _check_all_rows(p)


def test_backward_closed_form_sums_and_determinism(dev):
    """Per head, the dV rows add up to the dO rows' sum and the dK rows to
    zero (within the rounding of the bf16 gradients); two calls give the same
    bits."""
    p = isa.Params(1, 4, 1500, 1300, 128, 64, 0.25, 0.5, 0.125)
    inp = isa_inputs.make_inputs(STREAM["tiny"], p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, 3)
    r1 = _run(p, inp, dO_bits, dev)
    r2 = _run(p, inp, dO_bits, dev)
    for k in ("dQ", "dK", "dV"):
        assert np.array_equal(r1[k], r2[k]), k
    for h in range(p.H):
        sv, so = r1["dV"][0, h].sum(0), dO_vals[0, h].sum(0)
        sk = r1["dK"][0, h].sum(0)
        scale_v = np.abs(r1["dV"][0, h]).sum(0)
        scale_k = np.abs(r1["dK"][0, h]).sum(0)
        log(f"head {h}: |sum dV - sum dO| max {np.abs(sv - so).max():.3e}; |sum dK| max {np.abs(sk).max():.3e}")
        assert (np.abs(sv - so) <= 0.02 * scale_v + 1e-3).all()
        assert (np.abs(sk) <= 0.02 * scale_k + 1e-3).all()


@pytest.mark.parametrize("gamma,D,b", [(0.5, 128, 64), (-0.3, 64, 32)])
def test_backward_with_residual(dev, gamma, D, b):
    """gamma != 0: the residual gamma * O_coarse adds its gradient through the
    block means (oracle R12); every element against the oracle."""
    p = isa.Params(1, 2, 700, 451, D, b, 0.25, 0.5, 0.125, gamma)
    _check_all_rows(p)


def test_backward_residual_sums(dev):
    """With the residual the dV rows add up to (1 + gamma) times the summed dO
    rows (each coarse softmax row sums to one too)."""
    gamma = 0.4
    p = isa.Params(1, 2, 1500, 1300, 128, 64, 0.25, 0.5, 0.125, gamma)
    inp = isa_inputs.make_inputs(STREAM["tiny"], p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, 4)
    r = _run(p, inp, dO_bits, dev)
    for h in range(p.H):
        sv, so = r["dV"][0, h].sum(0), (1 + gamma) * dO_vals[0, h].sum(0)
        log(f"head {h}: |sum dV - (1+gamma) sum dO| max {np.abs(sv - so).max():.3e}")
        assert (np.abs(sv - so) <= 0.02 * np.abs(r["dV"][0, h]).sum(0) + 1e-3).all()


def test_backward_with_rope_and_residual(dev):
    """RoPE and the residual together (b = 32, D = 64): every gradient of the
    unrotated Q, K and of V against the oracle."""
    p = isa.Params(1, 2, 700, 451, 64, 32, 0.25, 0.5, 0.125, 0.3, rope_base=10000.0)
    _check_all_rows(p)


def test_backward_with_rope(dev):
    """RoPE on: the gradients of the unrotated Q, K (oracle: the backward on
    the rotated tensors, then the transposed rotation)."""
    p = isa.Params(1, 2, 700, 451, 128, 64, 0.25, 0.5, 0.125, rope_base=10000.0)
    _check_all_rows(p)


def test_backward_16k_workload(dev):
    """16K-token workload (H = 40, D = 128, b = 64, default ratios): two heads
    against the oracle element by element, every head through the sums."""
    c = isa_inputs.WORKLOADS["16k"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"])
    log("16k backward")
    res, _ = _check_all_rows(p, stream=STREAM["16k"], heads=[(0, 0), (0, 39)])
    _, dO_vals = _dO(p, 0)
    for h in range(p.H):
        sv, so, sk = res["dV"][0, h].sum(0), dO_vals[0, h].sum(0), res["dK"][0, h].sum(0)
        assert (np.abs(sv - so) <= 0.02 * np.abs(res["dV"][0, h]).sum(0) + 1e-3).all(), h
        assert (np.abs(sk) <= 0.02 * np.abs(res["dK"][0, h]).sum(0) + 1e-3).all(), h


def test_backward_64k_workload(dev):
    """The 64K-token workload (H = 40, D = 128, b = 64, default ratios) in the
    launch configuration the benchmark times: dQ of sampled rows (segment and
    tail edges included) of three heads against the oracle row by row, and
    the gradient sums of every head."""
    c = isa_inputs.WORKLOADS["64k"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"])
    inp = isa_inputs.make_inputs(STREAM["64k"], p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, 9)
    log("64k backward")
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    dO = bf16_tensor(dO_bits, dev)
    ws = isa.workspace(p, dev)
    O, dbg = isa.forward(Q, K, V, p, debug=True, workspace=ws)
    dQ, dK, dV = isa.backward(Q, K, V, O, dO, p, ws)
    torch.cuda.synchronize()
    sv = dV.float().sum(dim=2)[0]
    sk = dK.float().sum(dim=2)[0]
    av = dV.float().abs().sum(dim=2)[0]
    ak = dK.float().abs().sum(dim=2)[0]
    so = dO.float().sum(dim=2)[0]
    assert bool(((sv - so).abs() <= 0.02 * av + 1e-3).all())
    assert bool((sk.abs() <= 0.02 * ak + 1e-3).all())
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    sel = {k: v.cpu().numpy() for k, v in dbg.items()}
    rng = np.random.default_rng(21)
    for h in (0, 17, 39):
        rows = set(rng.choice(plan.L_src + plan.L_ctx, size=160, replace=False).tolist())
        rows |= {0, plan.L_src - 1, plan.L_src, plan.L_src + plan.L_ctx - 1}
        rows = np.array(sorted(rows))
        Qv, Kv, Vv = (inp[n][1][0, h] for n in "QKV")
        own = isa_oracle.isa_head(Qv, Kv, Vv, plan, compute_output=False)
        assert np.array_equal(own.ctx_idx + plan.N_src, sel["ctx_idx"][0, h])
        assert np.array_equal(own.sharp_idx, sel["sharp_idx"][0, h])
        assert np.array_equal(own.flat_exact_idx, sel["flat_exact_idx"][0, h])
        ref = isa_oracle.isa_head_dq_rows(Qv, Kv, Vv, dO_vals[0, h], plan, rows)
        got = dQ[0, h, torch.from_numpy(rows).to(dev)].float().cpu().numpy()
        log(f"head {h}")
        _compare("dQ rows", got, ref)


def test_backward_block_shared_by_every_exact_set(dev):
    """One kept block that every flat block reads exactly (every query shares
    a component its keys point along): its list of flat blocks holds all of
    them, the longest the backward's inverse lists can get. Every gradient
    element against the oracle."""
    p = isa.Params(1, 2, 6400, 6400, 64, 64, 0.25, 0.5, 0.125)
    inp = isa_inputs.make_inputs(STREAM["tiny"], p.B, p.H, p.L_src, p.L_ctx, p.D)
    rng = np.random.default_rng(123)
    for h in range(p.H):
        u = rng.standard_normal(p.D).astype(np.float32)
        u /= np.linalg.norm(u)
        q = inp["Q"][1][0, h].astype(np.float32) + 2.0 * u[None, :]    # a component every query shares
        k = inp["K"][1][0, h].astype(np.float32).copy()
        k[:64] = 6.0 * u[None, :] + 0.1 * k[:64]                        # block 0 points along it
        for name, x in (("Q", q), ("K", k)):
            bits, val = isa_inputs.round_to_bf16(x)
            inp[name][0][0, h] = bits
            inp[name][1][0, h] = val
    dO_bits, dO_vals = _dO(p, 5)
    res = _run(p, inp, dO_bits, dev)
    E = res["sel"]["flat_exact_idx"]
    assert (E[0] == 0).any(axis=-1).all(), "block 0 must be in every exact set"
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        log(f"head {h}")
        gq, gk, gv = _oracle_grads(plan, inp, dO_vals, 0, h, res["sel"])
        _compare("dQ", res["dQ"][0, h], gq)
        _compare("dK", res["dK"][0, h], gk)
        _compare("dV", res["dV"][0, h], gv)


@pytest.mark.parametrize("L_src,L_ctx,b,a_s,a_f,a_ns", [
    (40, 0, 64, 0.25, 0.5, 0.25),    # one partial block, no context
    (1, 70, 32, 0.5, 0.5, 0.5),      # a one-token source segment
    (65, 1, 64, 1.0, 0.5, 0.5),      # one-token tails in both segments
    (33, 97, 32, 0.34, 0.7, 0.2),    # one-token tails, one exact block per flat block
])
def test_forward_backward_tiny_edges(dev, L_src, L_ctx, b, a_s, a_f, a_ns):
    """Degenerate shapes: forward (every row) and backward (every gradient)
    against the oracle."""
    p = isa.Params(1, 2, L_src, L_ctx, 64, b, a_s, a_f, a_ns)
    inp = isa_inputs.make_inputs(STREAM["tiny"], p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, 6)
    res = _run(p, inp, dO_bits, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        r = isa_oracle.isa_head(*(inp[n][1][0, h] for n in "QKV"), plan)
        e = np.abs(res["O"][0, h] - r.O)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3, (h, e.max(), e.mean())
        gq, gk, gv = _oracle_grads(plan, inp, dO_vals, 0, h, res["sel"])
        _compare("dQ", res["dQ"][0, h], gq)
        _compare("dK", res["dK"][0, h], gk)
        _compare("dV", res["dV"][0, h], gv)


def _random_cases(n=24, seed=2024, max_len=1200, max_b=2, max_h=3):
    """Seeded draws over the whole parameter space: batch and heads, lengths
    (ragged, and L_ctx = 0), D, b, the three ratios with their edge values,
    gamma and RoPE."""
    rng = np.random.default_rng(seed)
    pick = lambda xs: xs[int(rng.integers(len(xs)))]
    ratio = lambda: float(pick([0.0, 1.0, round(float(rng.uniform()), 3), round(float(rng.uniform()), 3)]))
    cases = []
    for k in range(n):
        L_src = int(rng.integers(1, max_len))
        L_ctx = int(pick([0, int(rng.integers(1, max_len)), int(rng.integers(1, max_len))]))
        cases.append(dict(B=int(rng.integers(1, max_b + 1)), H=int(rng.integers(1, max_h + 1)),
                          L_src=L_src, L_ctx=L_ctx,
                          D=int(pick([64, 128])), b=int(pick([32, 64])), a_s=ratio(), a_f=ratio(),
                          a_ns=ratio(), gamma=float(pick([0.0, 0.0, 0.4, -0.3])),
                          rope=float(pick([0.0, 10000.0]))))
    return cases


# 24 draws of up to 1200 tokens per segment, and 12 longer ones (up to 3000,
# one batch, at most two heads, so that the fp64 oracle stays in seconds)
RANDOM_CASES = (list(enumerate(_random_cases()))
                + [(100 + k, c) for k, c in enumerate(_random_cases(12, 7, 3000, 1, 2))])


@pytest.mark.parametrize("k,c", RANDOM_CASES)
def test_random_shapes_forward_backward(dev, k, c):
    """Seeded random shapes and options: the forward over every row (selections
    checked up to the tie band) and every gradient element. The oracle's
    backward runs on its own selections; a head whose selections differ
    inside the tie band (its gradients then have no unique expected value)
    is left out of the gradient check, and every case compares at least one
    head."""
    from parity_util import compare_head
    log(f"random case {k}: {c}")
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"], c["a_s"], c["a_f"], c["a_ns"],
                   c["gamma"], c["rope"])
    inp = isa_inputs.make_inputs(1000 + k, p.B, p.H, p.L_src, p.L_ctx, p.D)
    dO_bits, dO_vals = _dO(p, 100 + k)
    res = _run(p, inp, dO_bits, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    graded = 0
    for bi in range(p.B):
        for h in range(p.H):
            Qv, Kv, Vv = (inp[n][1][bi, h] for n in "QKV")
            if p.rope_base:
                Qv = isa_oracle.rope(Qv, plan.L_src, plan.L_ctx, p.rope_base)
                Kv = isa_oracle.rope(Kv, plan.L_src, plan.L_ctx, p.rope_base)
            gpu = {name: res["sel"][name][bi, h] for name in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx")}
            gpu["O"] = res["O"][bi, h]
            rep = compare_head(plan, Qv, Kv, Vv, gpu,
                               oracle_result=isa_oracle.isa_head(Qv, Kv, Vv, plan, gamma=p.gamma))
            log(f"  head ({bi},{h}) forward max-abs {rep['max_abs']:.2e} excused {rep['excused']}")
            if rep["excused"]:
                log("  a selection lies inside the tie band: gradients of this head not compared")
                continue
            gq, gk, gv = isa_oracle.isa_head_backward(Qv, Kv, Vv, dO_vals[bi, h], plan, gamma=p.gamma)
            if p.rope_base:
                gq = isa_oracle.rope_backward(gq, plan.L_src, plan.L_ctx, p.rope_base)
                gk = isa_oracle.rope_backward(gk, plan.L_src, plan.L_ctx, p.rope_base)
            _compare("dQ", res["dQ"][bi, h], gq)
            _compare("dK", res["dK"][bi, h], gk)
            _compare("dV", res["dV"][bi, h], gv)
            graded += 1
    assert graded > 0, "every head of this case was excused"


def test_element_offsets_beyond_32_bits(dev):
    """H = 160 heads of 131072 tokens at D = 128: 2.7e9 elements (5.4 GB) per
    tensor, so the heads from 128 on start past element 2^31 and byte 2^32.
    Heads 0, 130 and 159 hold generated data (the others zeros); for each,
    every selection and sampled output rows against the oracle, the
    closed-form gradient sums, and dQ of the sampled rows."""
    from parity_util import compare_head
    Ls = Lc = 65536
    D, b, H = 128, 64, 160
    L = Ls + Lc
    checked = (0, 130, 159)
    assert checked[1] * L * D > 2 ** 31 and H * L * D * 2 > 2 ** 32
    p = isa.Params(1, H, Ls, Lc, D, b, 0.125, 0.5, 0.0625)
    plan = isa_oracle.make_plan(Ls, Lc, b, p.alpha_s, p.alpha_f, p.alpha_ns)
    log(f"offsets past 2^31: H={H} L={L} D={D} ({H * L * D / 1e9:.2f}e9 elements per tensor)")
    Q, K, V, dO = (torch.zeros(1, H, L, D, dtype=torch.bfloat16, device=dev) for _ in range(4))
    host = {}
    rng = np.random.default_rng(77)
    for h in checked:
        qkv = [isa_inputs.round_to_bf16(x) for x in isa_inputs.make_head(9, 0, h, Ls, Lc, D)]
        go = isa_inputs.round_to_bf16(rng.standard_normal((L, D)).astype(np.float32))
        for t, (bits, _) in zip((Q, K, V, dO), qkv + [go]):
            t[0, h].copy_(bf16_tensor(bits, dev))
        host[h] = ([v for _, v in qkv], go[1])
    ws = isa.workspace(p, dev)
    O, dbg = isa.forward(Q, K, V, p, debug=True, workspace=ws)
    dQ, dK, dV = isa.backward(Q, K, V, O, dO, p, ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    for h in checked:
        (Qv, Kv, Vv), dO_vals = host[h]
        r = np.random.default_rng([34, h])
        rows = np.array(sorted(set(r.choice(L, size=24, replace=False).tolist()) | {0, Ls - 1, Ls, L - 1}))
        gpu = {k: dbg[k][0, h].cpu().numpy() for k in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx")}
        gpu["O"] = f(O[0, h])
        rep = compare_head(plan, Qv, Kv, Vv, gpu, rows=rows)
        log(f"  head {h}: max-abs {rep['max_abs']:.2e} mean-abs {rep['mean_abs']:.2e} excused {rep['excused']}")
        gv, gk = f(dV[0, h]), f(dK[0, h])
        sv, sk, so = gv.sum(0), gk.sum(0), dO_vals.astype(np.float64).sum(0)
        assert (np.abs(sv - so) <= 0.02 * np.abs(gv).sum(0) + 1e-3).all()
        assert (np.abs(sk) <= 0.02 * np.abs(gk).sum(0) + 1e-3).all()
        if rep["excused"]:
            log("  a selection lies inside the tie band: dQ rows not compared")
            continue
        ref = isa_oracle.isa_head_dq_rows(Qv, Kv, Vv, dO_vals, plan, rows)
        _compare(f"head {h} dQ rows", f(dQ[0, h])[rows], ref)


def test_maximum_block_counts(dev):
    """The largest block counts the library accepts: N_kv = 4096 kept blocks
    (all 3584 source blocks and 512 of the 4096 context blocks, the last one
    partial), b = 32, D = 64, k_ns = 256 exact blocks per flat block. Every
    selection and sampled output rows against the oracle, the closed-form
    gradient sums, and dQ of the sampled rows."""
    from parity_util import compare_head
    Ls, Lc, D, b = 3584 * 32, 4096 * 32 - 5, 64, 32
    p = isa.Params(1, 1, Ls, Lc, D, b, 0.125, 0.5, 0.0625)
    pl = isa.plan(p)
    assert pl["N_kv"] == 4096 and pl["N_ctx"] == 4096 and pl["N_src"] == 3584 and pl["k_ns"] == 256
    log("maximum block counts: inputs")
    inp = isa_inputs.make_inputs(7, p.B, p.H, Ls, Lc, D)
    dO_bits, dO_vals = _dO(p, 12)
    res = _run(p, inp, dO_bits, dev)
    plan = isa_oracle.make_plan(Ls, Lc, b, p.alpha_s, p.alpha_f, p.alpha_ns)
    L = Ls + Lc
    rng = np.random.default_rng(33)
    rows = np.array(sorted(set(rng.choice(L, size=40, replace=False).tolist()) | {0, Ls - 1, Ls, L - 5, L - 1}))
    Qv, Kv, Vv = (inp[n][1][0, 0] for n in "QKV")
    gpu = {name: res["sel"][name][0, 0] for name in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx")}
    gpu["O"] = res["O"][0, 0]
    log("maximum block counts: oracle")
    rep = compare_head(plan, Qv, Kv, Vv, gpu, rows=rows)
    log(f"  forward: max-abs {rep['max_abs']:.2e} mean-abs {rep['mean_abs']:.2e} excused {rep['excused']}")
    sv, sk, so = res["dV"][0, 0].sum(0), res["dK"][0, 0].sum(0), dO_vals[0, 0].astype(np.float64).sum(0)
    av, ak = np.abs(res["dV"][0, 0]).sum(0), np.abs(res["dK"][0, 0]).sum(0)
    assert (np.abs(sv - so) <= 0.02 * av + 1e-3).all() and (np.abs(sk) <= 0.02 * ak + 1e-3).all()
    if rep["excused"]:
        log("  a selection lies inside the tie band: dQ rows not compared")
        return
    ref = isa_oracle.isa_head_dq_rows(Qv, Kv, Vv, dO_vals[0, 0], plan, rows)
    _compare("dQ rows", res["dQ"][0, 0][rows], ref)


def test_backward_reads_no_row_of_out_of_range_block_ids(dev):
    """isa_backward takes the selections the forward saved in the workspace.
    On a workspace no forward filled (every word -1), every block id it reads
    is out of range: such ids give empty token ranges, so the call reads no
    row outside the tensors and completes; a forward then refills the
    workspace and the backward gives the usual gradients."""
    p = isa.Params(1, 2, 700, 451, 128, 64, 0.25, 0.5, 0.125)
    inp = isa_inputs.make_inputs(1, p.B, p.H, p.L_src, p.L_ctx, p.D)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    dO_bits, _ = _dO(p, 3)
    dO = bf16_tensor(dO_bits, dev)
    O = torch.zeros_like(Q)
    ws = isa.workspace(p, dev)
    ws.fill_(255)
    log("backward on a workspace of -1 words")
    isa.backward(Q, K, V, O, dO, p, ws)
    torch.cuda.synchronize()
    O = isa.forward(Q, K, V, p, workspace=ws)
    dQ, dK, dV = isa.backward(Q, K, V, O, dO, p, ws)
    ws2 = isa.workspace(p, dev)
    O2 = isa.forward(Q, K, V, p, workspace=ws2)
    ref = isa.backward(Q, K, V, O2, dO, p, ws2)
    torch.cuda.synchronize()
    for a, b in zip((dQ, dK, dV), ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
