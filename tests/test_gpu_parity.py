"""GPU parity of the HIP ISA path against the CPU oracle, through the C ABI.

Small shapes compare every output element; the full workload shapes compare
every selection of every head and sampled output rows of a few heads (the
oracle computes those rows one by one). Special cases of the method are
re-checked on the GPU."""
from __future__ import annotations

import sys
import time

import numpy as np
import pytest

import isa_inputs
from oracle import isa_oracle
from parity_util import OraclePool, bf16_tensor, compare_head

STREAM = {name: w["stream"] for name, w in isa_inputs.WORKLOADS.items()}

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
isa = pytest.importorskip("block_sparse_attention_blockwise_amd")


def log(msg):
    print(f"[gpu-parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    isa.lib()
    return torch.device("cuda:0")


def _inputs(stream, p, heads=None, tile_heads=False):
    """bf16 inputs [B,H,L,D]. With tile_heads, only `heads` are generated and
    copied round-robin into the other head slots (the launch shape stays the
    full one; only the listed heads are checked)."""
    if not tile_heads:
        return isa_inputs.make_inputs(stream, p.B, p.H, p.L_src, p.L_ctx, p.D)
    gen = isa_inputs.make_inputs(stream, p.B, p.H, p.L_src, p.L_ctx, p.D, heads=heads)
    for nm in "QKV":
        bits, val = gen[nm]
        for bi in range(p.B):
            for h in range(p.H):
                if (bi, h) not in heads:
                    src = heads[h % len(heads)]
                    bits[bi, h] = bits[src]
                    val[bi, h] = val[src]
    return gen


def _run(p, inp, dev):
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    O, dbg = isa.forward(Q, K, V, p, debug=True)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in dbg.items()}
    out["O"] = O.float().cpu().numpy()
    return out


def _gpu_head(res, bi, h):
    return {k: res[k][bi, h] for k in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx", "O")}


def _sample_rows(plan, n, seed):
    rng = np.random.default_rng(seed)
    L = plan.L_src + plan.L_ctx
    rows = set(rng.choice(L, size=min(n, L), replace=False).tolist())
    # first and last rows of both segments, and of the tail blocks
    for t in (0, plan.L_src - 1, plan.L_src, L - 1, plan.starts[plan.N_src - 1], plan.starts[-1]):
        rows.add(int(t))
    return np.array(sorted(rows))


def _check(p, inp, res, out_heads, rows_per_head, seed=0, all_sel=True):
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    heads = [(bi, h) for bi in range(p.B) for h in range(p.H)] if all_sel else list(out_heads)
    worst = 0.0
    for (bi, h) in heads:
        Qv, Kv, Vv = (inp[n][1][bi, h] for n in "QKV")
        if (bi, h) in out_heads:
            rows = None if rows_per_head is None else _sample_rows(plan, rows_per_head, seed + h)
            rep = compare_head(plan, Qv, Kv, Vv, _gpu_head(res, bi, h), rows=rows)
            worst = max(worst, rep["max_abs"])
            log(f"  head ({bi},{h}): max-abs {rep['max_abs']:.2e} mean-abs {rep['mean_abs']:.2e} "
                f"rel-L2 {rep['rel_l2']:.2e} rows {rep['n_compared'] // p.D} "
                f"(skipped {rep['n_rows_skipped']}) excused {rep['excused']}")
            assert rep["n_compared"] > 0, f"head ({bi},{h}): no output row compared"
        else:
            # selections only
            compare_head(plan, Qv, Kv, Vv, _gpu_head(res, bi, h), rows=np.zeros(0, dtype=np.int64))
    return worst


@pytest.fixture(scope="module")
def pool():
    with OraclePool() as pl:
        yield pl


def _gpu_inputs(stream, p, dev, gen_heads=None):
    """Device Q, K, V [B,H,L,D] bf16 of the seeded generator. With gen_heads,
    only those heads are generated and the other head slots repeat them
    round-robin (the launch keeps its full shape)."""
    L = p.L_src + p.L_ctx
    T = [torch.empty((p.B, p.H, L, p.D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    heads = gen_heads or [(bi, h) for bi in range(p.B) for h in range(p.H)]
    for (bi, h) in heads:
        qkv = isa_inputs.make_head(stream, bi, h, p.L_src, p.L_ctx, p.D)
        for t, x in zip(T, qkv):
            t[bi, h].copy_(bf16_tensor(isa_inputs.round_to_bf16(x)[0], dev))
    if gen_heads:
        for bi in range(p.B):
            for h in range(p.H):
                if (bi, h) not in gen_heads:
                    src = gen_heads[h % len(gen_heads)]
                    for t in T:
                        t[bi, h].copy_(t[src])
    return T


def _check_pool(pool, stream, p, Q, K, V, full_heads=(), sampled_heads=(), rows_per_head=0,
                seed=0, sel_heads=None):
    """Runs the forward and compares with the oracle in worker processes:
    every row of `full_heads`, sampled rows of `sampled_heads`, and the
    selections of `sel_heads` (default: every head). Heads are regenerated
    by the workers from the seed `stream`."""
    O, dbg = isa.forward(Q, K, V, p, debug=True)
    torch.cuda.synchronize()
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    sel = {k: v.cpu().numpy() for k, v in dbg.items()}
    all_heads = [(bi, h) for bi in range(p.B) for h in range(p.H)]
    heads = list(dict.fromkeys(list(full_heads) + list(sampled_heads) +
                               list(all_heads if sel_heads is None else sel_heads)))
    jobs = []
    for (bi, h) in heads:
        gpu = {k: sel[k][bi, h] for k in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx")}
        if (bi, h) in full_heads:
            rows = None
            gpu["O"] = O[bi, h].float().cpu().numpy()
        elif (bi, h) in sampled_heads:
            rows = _sample_rows(plan, rows_per_head, seed + h)
            gpu["O_rows"] = O[bi, h, torch.from_numpy(rows).to(O.device)].float().cpu().numpy()
        else:
            rows = np.zeros(0, dtype=np.int64)
        jobs.append(dict(stream=stream, bi=bi, h=h, L_src=p.L_src, L_ctx=p.L_ctx, D=p.D, b=p.b,
                         ratios=(p.alpha_s, p.alpha_f, p.alpha_ns), gpu=gpu, rows=rows))
    del O
    out_heads = set(full_heads) | set(sampled_heads)
    worst, n_rows = 0.0, 0
    for job, rep in zip(jobs, pool.run(jobs)):
        hd = (job["bi"], job["h"])
        if hd in out_heads:
            assert rep["n_compared"] > 0, f"head {hd}: no output row compared"
            worst = max(worst, rep["max_abs"])
            n_rows += rep["n_compared"] // p.D
            log(f"  head {hd}: max-abs {rep['max_abs']:.2e} mean-abs {rep['mean_abs']:.2e} "
                f"rel-L2 {rep['rel_l2']:.2e} rows {rep['n_compared'] // p.D} "
                f"(skipped {rep['n_rows_skipped']}) excused {rep['excused']}")
        elif rep["excused"]:
            log(f"  head {hd}: selections excused {rep['excused']}")
    log(f"  {len(jobs)} heads' selections, {n_rows} output rows compared; worst max-abs {worst:.2e}")
    return worst


# ------------------------------------------------------------- workloads
def test_tiny_all_rows(dev):
    c = isa_inputs.WORKLOADS["tiny"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"])
    inp = _inputs(STREAM["tiny"], p)
    log("tiny: forward")
    res = _run(p, inp, dev)
    _check(p, inp, res, {(0, 0), (0, 1)}, None)


# every row of these heads (all 40 at 16384 tokens), every selection of every head
FULL_ROW_HEADS = {"16k": [(0, h) for h in range(40)],
                  "23768_ragged": [(0, h) for h in (0, 7, 17, 23, 31, 39)],
                  "64k": [(0, h) for h in (0, 13, 26, 39)]}


@pytest.mark.parametrize("name", ["16k", "23768_ragged", "64k"])
def test_workloads(dev, pool, name):
    c = isa_inputs.WORKLOADS[name]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"])
    log(f"{name}: generating inputs")
    Q, K, V = _gpu_inputs(c["stream"], p, dev)
    log(f"{name}: forward; every selection of {p.H} heads, every row of {len(FULL_ROW_HEADS[name])}")
    _check_pool(pool, c["stream"], p, Q, K, V, full_heads=FULL_ROW_HEADS[name])


# the 131072-token grid: every (b, alpha_s, alpha_ns, alpha_f) point
SWEEP = [(b, a_s, a_ns, a_f) for b in (64, 32) for a_s in (0.125, 0.25) for a_ns in (0.0625, 0.125)
         for a_f in (0.25, 0.5, 0.75)]
SWEEP_HEADS = [(0, 3), (0, 29)]


@pytest.fixture(scope="module")
def inputs_128k(dev):
    c = isa_inputs.WORKLOADS["128k"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"])
    log("128k: generating two heads, tiled over 40")
    return _gpu_inputs(c["stream"], p, dev, gen_heads=SWEEP_HEADS)


@pytest.mark.parametrize("b,a_s,a_ns,a_f", SWEEP)
def test_128k_sweep_points(dev, pool, inputs_128k, b, a_s, a_ns, a_f):
    """Full H = 40 launch at 131072 tokens; both generated heads: every
    selection and sampled output rows against the oracle."""
    c = isa_inputs.WORKLOADS["128k"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], b, a_s, a_f, a_ns)
    log(f"128k b={b} a_s={a_s} a_ns={a_ns} a_f={a_f}: forward")
    Q, K, V = inputs_128k
    _check_pool(pool, c["stream"], p, Q, K, V, sampled_heads=SWEEP_HEADS, rows_per_head=128, seed=b,
                sel_heads=SWEEP_HEADS)


# -------------------------------------------------------- special cases
def _small(dev, L_src, L_ctx, D, b, a_s, a_f, a_ns, H=2, stream=1, modify=None):
    p = isa.Params(1, H, L_src, L_ctx, D, b, a_s, a_f, a_ns)
    inp = _inputs(stream, p)
    if modify:
        modify(inp, p)
    res = _run(p, inp, dev)
    return p, inp, res


@pytest.mark.parametrize("D,b", [(128, 64), (64, 32), (128, 32), (64, 64)])
def test_small_shapes_all_rows(dev, D, b):
    p, inp, res = _small(dev, 700, 451, D, b, 0.25, 0.5, 0.125)
    _check(p, inp, res, {(0, 0), (0, 1)}, None)


@pytest.mark.parametrize("D", [64, 128])
def test_flat_key_half_without_keys(dev, D):
    """b = 32 flat blocks split each 64-key tile between two wave pairs. With
    N_kv = 9 kept blocks and k_ns = 1, the second half of every tile is
    padding (one 32-token exact block; 9 pooled positions), so that half's
    softmax state stays empty and must merge with weight 0: every row."""
    p, inp, res = _small(dev, 256, 256, D, 32, 0.125, 0.5, 0.0625)
    pl = isa.plan(p)
    assert pl["N_kv"] == 9 and pl["k_ns"] == 1 and pl["n_flat"] > 0
    _check(p, inp, res, {(0, 0), (0, 1)}, None)


def test_flat_grid_order_with_distinct_heads(dev):
    """The 32-token flat kernel takes an XCD-contiguous grid order when its
    workgroup count is a multiple of 8. Here B*H = 8 distinct heads (no tiled
    copies), b = 32, a large exact set: every selection of every head and
    every output row of every head against the oracle."""
    p = isa.Params(2, 4, 1536, 1600, 128, 32, 0.25, 0.75, 0.25)
    pl = isa.plan(p)
    assert (pl["n_flat"] * p.B * p.H) % 8 == 0 and pl["k_ns"] > 1
    inp = _inputs(STREAM["23768_ragged"], p)
    res = _run(p, inp, dev)
    heads = {(bi, h) for bi in range(p.B) for h in range(p.H)}
    _check(p, inp, res, heads, None)


def test_flat_block_order_b64_distinct_heads(dev):
    """isa_forward runs the 64-token flat kernel in the grid order that the
    library ranks the flat blocks into (by the first block of their exact
    sets, each XCD taking a contiguous run when the workgroup count is a
    multiple of 8). Here B*H = 8 distinct heads, b = 64, a large exact set:
    every selection and every output row of every head against the oracle,
    and the stand-alone flat entry point (plain order) gives the same bits."""
    p = isa.Params(2, 4, 3072, 3200, 128, 64, 0.25, 0.75, 0.25)
    pl = isa.plan(p)
    assert (pl["n_flat"] * p.B * p.H) % 8 == 0 and pl["k_ns"] > 1
    inp = _inputs(STREAM["23768_ragged"], p)
    res = _run(p, inp, dev)
    heads = {(bi, h) for bi in range(p.B) for h in range(p.H)}
    _check(p, inp, res, heads, None)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    O_ref, dbg = isa.forward(Q, K, V, p, debug=True)
    _, _, kcb, vcb = isa.pool_coarse(Q, K, V, p)
    O = O_ref.clone()
    isa.flat_taylor_attn(Q, K, V, kcb, vcb, dbg["ctx_idx"], dbg["flat_idx"], dbg["flat_exact_idx"], p, out=O)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O_ref.view(torch.int16))


@pytest.mark.parametrize("B,H", [(2, 3), (3, 5)])
def test_batch_and_odd_head_counts(dev, B, H):
    """B > 1 and head counts that do not fill the XCD remap evenly."""
    p = isa.Params(B, H, 640, 520, 128, 64, 0.25, 0.5, 0.125)
    inp = _inputs(STREAM["16k"], p)
    res = _run(p, inp, dev)
    _check(p, inp, res, {(B - 1, H - 1), (0, 1)}, None)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    Od = isa.dense_attn(Q, K, V).float().cpu().numpy()
    for (bi, h) in ((0, 0), (B - 1, H - 1)):
        ref = isa_oracle.dense_attention(inp["Q"][1][bi, h], inp["K"][1][bi, h], inp["V"][1][bi, h])
        e = np.abs(Od[bi, h] - ref)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3


def test_dense_equality_and_dense_kernel(dev):
    for D in (64, 128):
        p, inp, res = _small(dev, 333, 410, D, 64, 1.0, 0.0, 0.0625)
        assert res["flat_idx"].size == 0
        Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
        Od = isa.dense_attn(Q, K, V).float().cpu().numpy()
        for h in range(p.H):
            ref = isa_oracle.dense_attention(inp["Q"][1][0, h], inp["K"][1][0, h], inp["V"][1][0, h])
            e1 = np.abs(res["O"][0, h] - ref)
            e2 = np.abs(Od[0, h] - ref)
            log(f"dense-equality D={D} h={h}: isa {e1.max():.2e} dense {e2.max():.2e}")
            for e in (e1, e2):
                assert e.max() <= 2e-2 and e.mean() <= 2e-3


@pytest.mark.parametrize("L,D", [(64, 128), (1000, 64), (4097, 128)])
def test_dense_kernel_ragged(dev, L, D):
    rng = np.random.default_rng(L)
    x = [isa_inputs.round_to_bf16(rng.standard_normal((1, 2, L, D)).astype(np.float32)) for _ in range(3)]
    Q, K, V = (bf16_tensor(b_, dev) for b_, _ in x)
    O = isa.dense_attn(Q, K, V).float().cpu().numpy()
    for h in range(2):
        ref = isa_oracle.dense_attention(x[0][1][0, h], x[1][1][0, h], x[2][1][0, h])
        e = np.abs(O[0, h] - ref)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3, (e.max(), e.mean())


def test_identical_keys_make_taylor_exact(dev):
    def flatten_keys(inp, p):
        plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, 0, 0, 0)
        bits, val = inp["K"]
        for s, n in zip(plan.starts, plan.counts):
            bits[:, :, s:s + n] = bits[:, :, s:s + 1]
            val[:, :, s:s + n] = val[:, :, s:s + 1]
    outs = []
    for a_ns in (0.0, 0.0625, 1.0):
        p, inp, res = _small(dev, 640, 576, 128, 64, 0.25, 0.5, a_ns, modify=flatten_keys)
        outs.append(res["O"])
    exact = isa_oracle.isa_head(inp["Q"][1][0, 0], inp["K"][1][0, 0], inp["V"][1][0, 0],
                                isa_oracle.make_plan(640, 576, 64, 0.25, 0.0, 0.0)).O
    for o in outs:
        e = np.abs(o[0, 0] - exact)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3


def test_kv_permutation_within_blocks(dev):
    p, inp, res = _small(dev, 768, 640, 128, 64, 0.25, 0.5, 0.125)
    plan = isa_oracle.make_plan(768, 640, 64, 0, 0, 0)
    rng = np.random.default_rng(5)
    inp2 = {n: (inp[n][0].copy(), inp[n][1].copy()) for n in "QKV"}
    for s, n in zip(plan.starts, plan.counts):
        perm = s + rng.permutation(n)
        for nm in "KV":
            inp2[nm][0][:, :, s:s + n] = inp[nm][0][:, :, perm]
            inp2[nm][1][:, :, s:s + n] = inp[nm][1][:, :, perm]
    res2 = _run(p, inp2, dev)
    for k in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx"):
        assert np.array_equal(res[k], res2[k]), k
    e = np.abs(res["O"] - res2["O"])
    assert e.max() <= 2e-2 and e.mean() <= 2e-3


def test_no_context_and_all_flat(dev):
    p, inp, res = _small(dev, 1000, 0, 128, 64, 0.125, 0.5, 0.0625)
    _check(p, inp, res, {(0, 0), (0, 1)}, None)
    p, inp, res = _small(dev, 500, 470, 64, 32, 1.0, 1.0, 0.0)
    assert res["sharp_idx"].size == 0
    _check(p, inp, res, {(0, 0), (0, 1)}, None)


def test_deterministic(dev):
    p, inp, res = _small(dev, 900, 700, 128, 64, 0.125, 0.5, 0.0625)
    res2 = _run(p, inp, dev)
    for k, v in res.items():
        assert np.array_equal(v, res2[k]), k


def test_step_entry_points_compose_to_forward(dev):
    c = isa_inputs.WORKLOADS["23768_ragged"]
    p = isa.Params(1, 4, c["L_src"], c["L_ctx"], c["D"], c["b"])
    inp = _inputs(STREAM["23768_ragged"], p)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    O_ref, dbg = isa.forward(Q, K, V, p, debug=True)
    qc, kc, kcb, vcb = isa.pool_coarse(Q, K, V, p)
    ctx, score = isa.ctx_topk(qc, kc, p)
    sharp, si, fi, ei = isa.sharpness_split(qc, kc, ctx, p)
    O = torch.zeros_like(Q)
    isa.sharp_attn(Q, K, V, ctx, si, p, out=O)
    isa.flat_taylor_attn(Q, K, V, kcb, vcb, ctx, fi, ei, p, out=O)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O_ref.view(torch.int16))
    for a, b in ((qc, "qc"), (kc, "kc"), (ctx, "ctx_idx"), (score, "ctx_score"), (sharp, "sharpness"),
                 (si, "sharp_idx"), (fi, "flat_idx"), (ei, "flat_exact_idx")):
        assert torch.equal(a, dbg[b]), b
    # pooled means are exact sums divided by n_j: bit-identical to the oracle
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        Qc = isa_oracle.pool(inp["Q"][1][0, h], plan)
        Kc = isa_oracle.pool(inp["K"][1][0, h], plan)
        assert np.array_equal(qc[0, h].cpu().numpy(), Qc)
        assert np.array_equal(kc[0, h].cpu().numpy(), Kc)
        S = isa_oracle.coarse_scores(Qc, Kc)
        M = isa_oracle.sharpness(S, plan)
        np.testing.assert_allclose(sharp[0, h].cpu().numpy(), M, rtol=1e-10, atol=0)
        r = isa_oracle.context_scores(S, plan)
        np.testing.assert_allclose(score[0, h].cpu().numpy(), r, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("gamma,D,b,Ls,Lc", [(0.5, 128, 64, 700, 451), (-0.25, 128, 64, 700, 451),
                                            (0.5, 64, 32, 1000, 1100)])
def test_coarse_residual_gamma(dev, gamma, D, b, Ls, Lc):
    """Step (6) residual: forward with gamma matches the oracle, and the
    residual entry point composes with the other steps. 19 and 67 query
    blocks: several 16-block workgroups of the residual kernel, the last
    one partial."""
    p = isa.Params(1, 2, Ls, Lc, D, b, 0.25, 0.5, 0.125, gamma)
    inp = _inputs(STREAM["tiny"], p)
    res = _run(p, inp, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        r = isa_oracle.isa_head(inp["Q"][1][0, h], inp["K"][1][0, h], inp["V"][1][0, h], plan, gamma=gamma)
        assert np.array_equal(res["sharp_idx"][0, h], r.sharp_idx)
        e = np.abs(res["O"][0, h] - r.O)
        log(f"residual gamma={gamma} h={h}: max-abs {e.max():.2e} mean-abs {e.mean():.2e}")
        assert e.max() <= 2e-2 and e.mean() <= 2e-3
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    p0 = isa.Params(1, 2, Ls, Lc, D, b, 0.25, 0.5, 0.125, 0.0)
    O0 = isa.forward(Q, K, V, p0)
    qc, kc, kcb, vcb = isa.pool_coarse(Q, K, V, p)
    ctx, _ = isa.ctx_topk(qc, kc, p)
    isa.coarse_residual(qc, kc, vcb, ctx, O0, p)
    Og = isa.forward(Q, K, V, p)
    torch.cuda.synchronize()
    assert torch.equal(O0.view(torch.int16), Og.view(torch.int16))


def test_pure_taylor_flat_path_at_16k(dev):
    """alpha_ns = 0: every flat block uses only the 0th-order Taylor terms
    (the variant the pages report as fastest). Full-size launch, selections of
    every head, sampled rows of three heads; then the Fig. 6 property on the
    GPU outputs: per-block Taylor error rises with sharpness."""
    from scipy.stats import spearmanr
    c = isa_inputs.WORKLOADS["16k"]
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"], 0.125, 1.0, 0.0)
    inp = _inputs(STREAM["16k"], p)
    log("pure Taylor 16k: forward")
    res = _run(p, inp, dev)
    assert res["sharp_idx"].size == 0
    _check(p, inp, res, {(0, 0), (0, 21), (0, p.H - 1)}, 256, seed=7)
    pe = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"], 0.125, 0.0, 0.0)
    exact = _run(pe, inp, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, 0.125, 1.0, 0.0)
    rhos = []
    for h in (0, 13, 39):
        err = [np.abs(res["O"][0, h, s_:s_ + n] - exact["O"][0, h, s_:s_ + n]).mean()
               for s_, n in zip(plan.starts, plan.counts)]
        rhos.append(spearmanr(res["sharpness"][0, h], err).correlation)
    log(f"Fig. 6 on GPU outputs: Spearman(sharpness, Taylor error) = {rhos}")
    assert min(rhos) > 0.5


# ------------------------------------------------------------ decoupled RoPE
def _bf16_bits_of(x):
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rope_mismatch(got_bits, want, X):
    """Counts rotated bf16 elements that differ from the oracle's. cos/sin
    come from different fp64 libms on the two sides (each within about an
    ulp), which can very rarely move an fp32 rounding of a table entry; such
    a difference stays within one bf16 ulp of the result plus one fp32 ulp of
    the pair's magnitude (the products can nearly cancel)."""
    w = _bf16_bits_of(want)
    bad = got_bits.astype(np.uint16) != w
    if bad.any():
        got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        X = np.asarray(X, dtype=np.float64)
        mag = np.repeat(np.abs(X[:, 0::2]) + np.abs(X[:, 1::2]), 2, axis=1)
        bound = 2.0 ** -7 * np.abs(want) + 2.0 ** -22 * mag
        assert (np.abs(got - want)[bad] <= bound[bad]).all()
    return int(bad.sum())


@pytest.mark.parametrize("D", [64, 128])
def test_rope_pool_matches_oracle(dev, D):
    """Rotated Q, K against the oracle's rotation (R11), element by element,
    and the pooled means of the rotated tensors."""
    base = 10000.0
    p = isa.Params(2, 3, 700, 451, D, 64, rope_base=base)
    inp = _inputs(STREAM["tiny"], p)
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    Qr, Kr, qc, kc, kcb, vcb = isa.rope_pool_coarse(Q, K, V, p)
    torch.cuda.synchronize()
    Qr_b = Qr.view(torch.int16).cpu().numpy().view(np.uint16)
    Kr_b = Kr.view(torch.int16).cpu().numpy().view(np.uint16)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    bad = 0
    for bi in range(p.B):
        for h in range(p.H):
            qr = isa_oracle.rope(inp["Q"][1][bi, h], p.L_src, p.L_ctx, base)
            kr = isa_oracle.rope(inp["K"][1][bi, h], p.L_src, p.L_ctx, base)
            bad += (_rope_mismatch(Qr_b[bi, h], qr, inp["Q"][1][bi, h])
                    + _rope_mismatch(Kr_b[bi, h], kr, inp["K"][1][bi, h]))
            np.testing.assert_allclose(qc[bi, h].cpu().numpy(), isa_oracle.pool(qr, plan),
                                       rtol=0, atol=1e-3)
            np.testing.assert_allclose(kc[bi, h].cpu().numpy(), isa_oracle.pool(kr, plan),
                                       rtol=0, atol=1e-3)
    total = 2 * p.B * p.H * (p.L_src + p.L_ctx) * D
    log(f"rope D={D}: {bad} of {total} rotated bf16 values differ from the oracle")
    assert bad <= total * 1e-5


def test_rope_forward_small_all_rows(dev):
    """Forward with RoPE against the oracle (rotation, then the method),
    every row; and bitwise equal to the forward without RoPE fed the rotated
    tensors of the RoPE entry point."""
    base = 10000.0
    p = isa.Params(1, 2, 700, 451, 128, 64, 0.25, 0.5, 0.125, rope_base=base)
    inp = _inputs(STREAM["tiny"], p)
    res = _run(p, inp, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        qr = isa_oracle.rope(inp["Q"][1][0, h], p.L_src, p.L_ctx, base)
        kr = isa_oracle.rope(inp["K"][1][0, h], p.L_src, p.L_ctx, base)
        rep = compare_head(plan, qr, kr, inp["V"][1][0, h], _gpu_head(res, 0, h))
        log(f"rope forward h={h}: max-abs {rep['max_abs']:.2e} excused {rep['excused']}")
    Q, K, V = (bf16_tensor(inp[n][0], dev) for n in "QKV")
    Qr, Kr, *_ = isa.rope_pool_coarse(Q, K, V, p)
    p0 = isa.Params(1, 2, 700, 451, 128, 64, 0.25, 0.5, 0.125)
    O0 = isa.forward(Qr, Kr, V, p0)
    Og = isa.forward(Q, K, V, p)
    torch.cuda.synchronize()
    assert torch.equal(O0.view(torch.int16), Og.view(torch.int16))


def test_rope_forward_ragged_workload(dev):
    """RoPE on the ragged 11884 + 11884-token workload (both segments end in
    a partial block; positions restart at the context segment): every
    selection of every head, sampled rows of two heads."""
    c = isa_inputs.WORKLOADS["23768_ragged"]
    base = 10000.0
    p = isa.Params(c["B"], c["H"], c["L_src"], c["L_ctx"], c["D"], c["b"], rope_base=base)
    inp = _inputs(STREAM["23768_ragged"], p)
    log("rope ragged workload: forward")
    res = _run(p, inp, dev)
    plan = isa_oracle.make_plan(p.L_src, p.L_ctx, p.b, p.alpha_s, p.alpha_f, p.alpha_ns)
    for h in range(p.H):
        qr = isa_oracle.rope(inp["Q"][1][0, h], p.L_src, p.L_ctx, base)
        kr = isa_oracle.rope(inp["K"][1][0, h], p.L_src, p.L_ctx, base)
        rows = _sample_rows(plan, 192, 11 + h) if h in (0, p.H - 1) else np.zeros(0, dtype=np.int64)
        rep = compare_head(plan, qr, kr, inp["V"][1][0, h], _gpu_head(res, 0, h), rows=rows)
        if rows.size:
            log(f"  head {h}: max-abs {rep['max_abs']:.2e} mean-abs {rep['mean_abs']:.2e} "
                f"excused {rep['excused']}")
