"""Pins for the CPU oracle: closed forms, special cases that reduce to a
library routine, invariants, brute force on tiny inputs and the figures the
pages print. Each test is chosen so that a plausible slip in the oracle (a
dropped term, a wrong index or sign, a transposed operand) fails it."""
import json
import math
import os

import numpy as np
import pytest
import torch

import isa_inputs
from oracle import isa_oracle as O
from oracle.brute import brute_isa_head

STREAM = {name: w["stream"] for name, w in isa_inputs.WORKLOADS.items()}

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_head(seed, L_src, L_ctx, D, spread=1.0):
    rng = np.random.default_rng(seed)
    L = L_src + L_ctx
    Q = rng.standard_normal((L, D))
    K = rng.standard_normal((L, D)) * spread
    V = rng.standard_normal((L, D))
    return Q, K, V


def _sdpa(q, k, v, mask=None):
    """CPU fp64 torch scaled_dot_product_attention (library routine)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(np.asarray(mask, dtype=np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)
    return out[0, 0].numpy()


# ------------------------------------------------------------------ counts
def test_counts_match_page_figures():
    g = json.load(open(os.path.join(HERE, "golden", "page_counts.json")))
    for L in (8192, 11884, 32768, 65536):
        p = O.make_plan(L, L, 64, g["alpha_s"], g["alpha_f"], g["alpha_ns"])
        if p.N_ctx % 8 == 0:
            assert 1 - p.k_ctx / p.N_ctx == g["context_pruned_fraction"]
        assert p.n_flat / p.N == g["taylor_query_fraction"]
        if p.N_kv % 16 == 0:
            assert 1 - p.k_ns / p.N_kv == g["taylor_path_sparsity"]


def test_counts_ragged_and_rounding():
    # 23768 tokens: 11884 = 185*64 + 44 per segment.
    p = O.make_plan(11884, 11884, 64, 0.125, 0.5, 0.0625)
    assert (p.N_src, p.N_ctx, p.N) == (186, 186, 372)
    assert p.counts[185] == 44 and p.counts[371] == 44 and p.counts[0] == 64
    assert p.starts[186] == 11884 and p.starts[185] == 185 * 64
    assert sum(p.counts) == 23768
    assert p.k_ctx == 24          # 0.125 * 186 = 23.25, rounded up
    assert p.N_kv == 210
    assert p.k_ns == 14           # 0.0625 * 210 = 13.125, rounded up
    assert (p.n_flat, p.n_sharp) == (186, 186)
    t = O.make_plan(1024, 1024, 64, 0.125, 0.5, 0.0625)
    assert (t.N, t.k_ctx, t.N_kv, t.k_ns, t.n_flat) == (32, 2, 18, 2, 16)
    h = O.make_plan(32768, 32768, 64, 0.125, 0.5, 0.0625)
    assert (h.N, h.k_ctx, h.N_kv, h.k_ns, h.n_flat) == (1024, 64, 576, 36, 512)
    e = O.make_plan(100, 0, 32, 0.125, 0.5, 0.0625)
    assert (e.N_src, e.N_ctx, e.k_ctx, e.counts) == (4, 0, 0, (32, 32, 32, 4))
    with pytest.raises(ValueError):
        O.make_plan(0, 10, 64, 0.1, 0.1, 0.1)
    with pytest.raises(ValueError):
        O.make_plan(10, 10, 64, 1.5, 0.1, 0.1)


# ------------------------------------------------------------------- pool
def test_pool_mean_and_permutation():
    p = O.make_plan(150, 70, 32, 0.5, 0.5, 0.5)
    rng = np.random.default_rng(0)
    X = rng.standard_normal((220, 8))
    P = O.pool(X, p)
    # explicit token loop, valid tokens only
    for j, (s, n) in enumerate(zip(p.starts, p.counts)):
        ref = [sum(X[t, d] for t in range(s, s + n)) / n for d in range(8)]
        assert np.allclose(P[j], ref, rtol=0, atol=1e-14)
    assert p.counts[4] == 22 and p.counts[-1] == 6
    Xp = X.copy()
    for s, n in zip(p.starts, p.counts):
        Xp[s:s + n] = Xp[s:s + n][rng.permutation(n)]
    assert np.allclose(O.pool(Xp, p), P, rtol=0, atol=1e-14)


# ------------------------------------------------------- context selection
def test_context_score_identity():
    p = O.make_plan(300, 260, 32, 0.25, 0.5, 0.1)
    Q, K, V = _rand_head(1, 300, 260, 16)
    Qc, Kc = O.pool(Q, p), O.pool(K, p)
    r = O.context_scores(O.coarse_scores(Qc, Kc), p)
    qbar = Qc[:p.N_src].sum(axis=0)
    r2 = (Kc[p.N_src:] @ qbar) / math.sqrt(16)
    assert np.allclose(r, r2, rtol=1e-12, atol=1e-12)
    # context query rows must not enter the score
    Qc2 = Qc.copy()
    Qc2[p.N_src:] *= 100.0
    assert np.allclose(O.context_scores(O.coarse_scores(Qc2, Kc), p), r, rtol=1e-12, atol=1e-12)


def test_top_k_ties_lowest_index():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, 0.0])
    assert list(O.top_k(s, 2)) == [1, 2]
    assert list(O.top_k(s, 3)) == [1, 2, 4]
    assert list(O.top_k(s, 4)) == [1, 2, 3, 4]
    assert list(O.top_k(s, 0)) == []
    assert list(O.top_k(np.zeros(5), 2)) == [0, 1]


# --------------------------------------------------------------- sharpness
def test_sharpness_closed_forms():
    p = O.make_plan(8 * 16, 8 * 16, 16, 0.5, 0.5, 0.5)  # N_src = 8, N = 16
    n = p.N_src
    S = np.zeros((p.N, p.N))
    S[1, 3] = 800.0                     # one-hot row over source columns
    S[2, n:] = np.arange(n) * 50.0      # spiky context columns only: ignored
    S[3, :n] = np.linspace(-1, 2, n)    # generic row
    M = O.sharpness(S, p)
    assert M[0] == pytest.approx(0.0, abs=1e-18)
    assert n * n * M[1] == pytest.approx(n - 1, rel=1e-12)
    assert M[2] == pytest.approx(0.0, abs=1e-18)
    x = np.exp(S[3, :n] - S[3, :n].max())
    pr = x / x.sum()
    assert M[3] == pytest.approx(np.var(pr), rel=1e-12)                # numpy population variance
    assert M[3] == pytest.approx(np.mean(pr ** 2) - 1 / n ** 2, rel=1e-9)  # Var = E[p^2] - 1/n^2


def test_split_extremes_and_ranking():
    rng = np.random.default_rng(3)
    M = rng.random(12)
    for af, ns in ((0.0, 12), (1.0, 0), (0.5, 6), (0.25, 9)):
        p = O.make_plan(6 * 4, 6 * 4, 4, 0.5, af, 0.5)
        sh, fl = O.split(M, p)
        assert len(sh) == ns and len(fl) == 12 - ns
        assert sorted(set(sh) | set(fl)) == list(range(12))
        if len(sh) and len(fl):
            assert M[sh].min() > M[fl].max()
    Mt = np.array([1.0, 2.0, 2.0, 2.0, 0.5, 1.0])
    p = O.make_plan(3 * 4, 3 * 4, 4, 0.5, 0.5, 0.5)
    sh, fl = O.split(Mt, p)
    assert list(sh) == [1, 2, 3] and list(fl) == [0, 4, 5]
    p2 = O.make_plan(3 * 4, 3 * 4, 4, 0.5, 4 / 6, 0.5)
    sh, fl = O.split(Mt, p2)
    assert list(sh) == [1, 2]   # tie among 1,2,3: lower index is sharper


# ------------------------------------------- whole path: special cases
@pytest.mark.parametrize("L_src,L_ctx,b,D", [(256, 256, 32, 16), (230, 170, 32, 8)])
def test_dense_equality(L_src, L_ctx, b, D):
    Q, K, V = _rand_head(5, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, 1.0, 0.0, 0.0625)
    r = O.isa_head(Q, K, V, p)
    assert len(r.flat_idx) == 0 and len(r.ctx_idx) == p.N_ctx
    ref = _sdpa(Q, K, V)
    assert np.abs(r.O - ref).max() < 1e-12
    assert np.abs(O.dense_attention(Q, K, V) - ref).max() < 1e-12


def test_no_context_equals_source_only_attention():
    Q, K, V = _rand_head(6, 192, 160, 8)
    p = O.make_plan(192, 160, 32, 0.0, 0.0, 0.5)
    r = O.isa_head(Q, K, V, p)
    assert np.abs(r.O - _sdpa(Q, K[:192], V[:192])).max() < 1e-12


def test_alpha_ns_one_is_exact_over_kept_blocks():
    Q, K, V = _rand_head(7, 200, 180, 8)
    a = O.isa_head(Q, K, V, O.make_plan(200, 180, 32, 0.5, 0.0, 0.0))
    b = O.isa_head(Q, K, V, O.make_plan(200, 180, 32, 0.5, 0.5, 1.0))
    assert len(b.flat_idx) > 0
    assert np.array_equal(a.ctx_idx, b.ctx_idx)
    assert np.abs(a.O - b.O).max() < 1e-12


def test_identical_keys_in_block_make_taylor_exact():
    L_src, L_ctx, b, D = 200, 150, 32, 8
    Q, K, V = _rand_head(8, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, 0.5, 0.5, 0.0)
    for s, n in zip(p.starts, p.counts):
        K[s:s + n] = K[s]
    outs = [O.isa_head(Q, K, V, O.make_plan(L_src, L_ctx, b, 0.5, 0.5, ans)).O
            for ans in (0.0, 0.0625, 0.3, 1.0)]
    exact = O.isa_head(Q, K, V, O.make_plan(L_src, L_ctx, b, 0.5, 0.0, 0.0)).O
    for o in outs:
        assert np.abs(o - exact).max() < 1e-12


def test_block_size_one_makes_taylor_exact():
    Q, K, V = _rand_head(9, 40, 30, 8)
    a = O.isa_head(Q, K, V, O.make_plan(40, 30, 1, 0.5, 0.5, 0.0)).O
    b = O.isa_head(Q, K, V, O.make_plan(40, 30, 1, 0.5, 0.0, 0.0)).O
    assert np.abs(a - b).max() < 1e-12


def test_pure_taylor_equals_pooled_sdpa_with_log_count_mask():
    L_src, L_ctx, b, D = 230, 170, 32, 8     # ragged tails: n_j varies
    Q, K, V = _rand_head(10, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, 1.0, 1.0, 0.0)
    r = O.isa_head(Q, K, V, p)
    assert len(r.sharp_idx) == 0 and p.k_ns == 0
    Kc, Vc = O.pool(K, p), O.pool(V, p)
    mask = np.log(np.asarray(p.counts, dtype=np.float64))[None, :].repeat(Q.shape[0], 0)
    ref = _sdpa(Q, Kc, Vc, mask)
    assert np.abs(r.O - ref).max() < 1e-12


def test_taylor_error_vanishes_with_key_spread():
    L_src, L_ctx, b, D = 128, 128, 16, 8
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((256, D))
    base = rng.standard_normal((16, D))
    noise = rng.standard_normal((256, D))
    V = rng.standard_normal((256, D))
    p = O.make_plan(L_src, L_ctx, b, 1.0, 1.0, 0.0)
    pe = O.make_plan(L_src, L_ctx, b, 1.0, 0.0, 0.0)
    errs = []
    for eps in (1e-1, 1e-2, 1e-3):
        K = np.repeat(base, 16, axis=0) + eps * noise
        errs.append(np.abs(O.isa_head(Q, K, V, p).O - O.isa_head(Q, K, V, pe).O).max())
    assert errs[0] > errs[1] > errs[2]
    # first order in the key spread: error ratio ~10 per decade
    assert 5 < errs[0] / errs[1] < 20 and 5 < errs[1] / errs[2] < 20


def test_kv_permutation_within_block_invariance():
    L_src, L_ctx, b, D = 224, 192, 32, 8
    Q, K, V = _rand_head(12, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, 0.5, 0.5, 0.25)
    ref = O.isa_head(Q, K, V, p)
    rng = np.random.default_rng(13)
    Kp, Vp, Qp = K.copy(), V.copy(), Q.copy()
    perm_q = np.arange(Q.shape[0])
    for s, n in zip(p.starts, p.counts):
        pk = rng.permutation(n)
        Kp[s:s + n], Vp[s:s + n] = K[s:s + n][pk], V[s:s + n][pk]
        pq = rng.permutation(n)
        perm_q[s:s + n] = s + pq
    out = O.isa_head(Q, Kp, Vp, p)
    assert np.abs(out.O - ref.O).max() < 1e-12
    outq = O.isa_head(Q[perm_q], K, V, p)
    assert np.abs(outq.O - ref.O[perm_q]).max() < 1e-12


# ------------------------------------------------------- brute force
@pytest.mark.parametrize("L_src,L_ctx,b,D,a_s,a_f,a_ns,seed", [
    (96, 160, 16, 8, 0.3, 0.5, 0.2, 21),
    (90, 150, 16, 8, 0.25, 0.5, 0.0625, 22),     # ragged tails
    (64, 64, 16, 4, 0.5, 0.75, 0.0, 23),
    (80, 0, 16, 4, 0.5, 0.5, 0.3, 24),           # no context
])
def test_blockwise_equals_brute_force(L_src, L_ctx, b, D, a_s, a_f, a_ns, seed):
    Q, K, V = _rand_head(seed, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, a_s, a_f, a_ns)
    r = O.isa_head(Q, K, V, p)
    g = brute_isa_head(Q, K, V, L_src, L_ctx, b, a_s, a_f, a_ns)
    assert np.array_equal(r.ctx_idx, g["ctx_idx"])
    assert np.array_equal(r.sharp_idx, g["sharp_idx"])
    assert np.array_equal(r.flat_idx, g["flat_idx"])
    assert np.array_equal(r.flat_exact_idx, g["flat_exact_idx"])
    assert np.abs(r.O - g["O"]).max() < 1e-12


def test_tiny_config_blockwise_equals_brute_force():
    c = isa_inputs.WORKLOADS["tiny"]
    Q, K, V = isa_inputs.make_head(STREAM["tiny"], 0, 0, c["L_src"], c["L_ctx"], c["D"])
    p = O.make_plan(c["L_src"], c["L_ctx"], c["b"], c["alpha_s"], c["alpha_f"], c["alpha_ns"])
    r = O.isa_head(Q, K, V, p)
    g = brute_isa_head(Q, K, V, c["L_src"], c["L_ctx"], c["b"], c["alpha_s"], c["alpha_f"], c["alpha_ns"])
    for k in ("ctx_idx", "sharp_idx", "flat_idx", "flat_exact_idx"):
        assert np.array_equal(getattr(r, k), g[k]), k
    assert np.abs(r.O - g["O"]).max() < 1e-12
    # both paths occur on the generator
    assert 0 < len(r.flat_idx) < p.N


def test_online_softmax_variant_matches_two_pass():
    """Block-by-block online softmax (running max, rescaled sums) over the
    same exact and Taylor terms equals the oracle's two-pass result."""
    L_src, L_ctx, b, D = 192, 160, 32, 8
    Q, K, V = _rand_head(30, L_src, L_ctx, D)
    p = O.make_plan(L_src, L_ctx, b, 0.5, 0.5, 0.25)
    r = O.isa_head(Q, K, V, p)
    J = O.kept_blocks(r.ctx_idx, p)
    s = 1 / math.sqrt(D)
    for rix, i in enumerate(r.flat_idx):
        t0, n = p.starts[i], p.counts[i]
        q = Q[t0:t0 + n]
        m = np.full(n, -np.inf)
        l = np.zeros(n)
        acc = np.zeros((n, D))
        for j in J:
            if j in r.flat_exact_idx[rix]:
                ks, vs = K[p.starts[j]:p.starts[j] + p.counts[j]], V[p.starts[j]:p.starts[j] + p.counts[j]]
                x = q @ ks.T * s
            else:
                ks, vs = r.Kc[j:j + 1], r.Vc[j:j + 1]
                x = q @ ks.T * s + math.log(p.counts[j])
            mn = np.maximum(m, x.max(axis=1))
            c = np.exp(m - mn)
            w = np.exp(x - mn[:, None])
            l = l * c + w.sum(axis=1)
            acc = acc * c[:, None] + w @ vs
            m = mn
        assert np.abs(acc / l[:, None] - r.O[t0:t0 + n]).max() < 1e-12


# --------------------------------------------------------------- soft
def test_taylor_error_grows_with_sharpness_soft():
    """Fig. 6 of the paper reports the per-block error of the 0th-order Taylor
    approximation rising with sharpness. Soft check (not a parity gate):
    positive rank correlation with every block on the pure Taylor path
    (alpha_ns = 0). With the default alpha_ns the exact set E_i absorbs the
    peak of sharp rows on this generator and the correlation turns negative;
    that case is not what the figure measures."""
    from scipy.stats import spearmanr
    c = isa_inputs.WORKLOADS["tiny"]
    Q, K, V = isa_inputs.make_head(STREAM["tiny"], 0, 1, c["L_src"], c["L_ctx"], c["D"])
    pt = O.make_plan(c["L_src"], c["L_ctx"], c["b"], c["alpha_s"], 1.0, 0.0)
    pe = O.make_plan(c["L_src"], c["L_ctx"], c["b"], c["alpha_s"], 0.0, 0.0)
    rt, re_ = O.isa_head(Q, K, V, pt), O.isa_head(Q, K, V, pe)
    err = [np.linalg.norm(rt.O[s:s + n] - re_.O[s:s + n]) for s, n in zip(pt.starts, pt.counts)]
    rho = spearmanr(rt.sharpness, err).correlation
    assert rho > 0.5


# ----------------------------------------------------------- generator
def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact halfway cases
    bits, val = isa_inputs.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(val, ref.float().numpy())


def test_generator_is_seeded_and_structured():
    a = isa_inputs.make_head(STREAM["64k"], 0, 3, 256, 256, 16)
    b = isa_inputs.make_head(STREAM["64k"], 0, 3, 256, 256, 16)
    c = isa_inputs.make_head(STREAM["64k"], 0, 4, 256, 256, 16)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])
    Q, K, V = a
    # context keys are scaled down
    assert np.abs(K[256:]).mean() < 0.7 * np.abs(K[:256]).mean()


# ------------------------------------------------- step (6) residual
def test_residual_off_by_default_and_linear_in_gamma():
    Q, K, V = _rand_head(40, 230, 170, 8)
    p = O.make_plan(230, 170, 32, 0.5, 0.5, 0.25)
    o0 = O.isa_head(Q, K, V, p).O
    assert np.array_equal(O.isa_head(Q, K, V, p, gamma=0.0).O, o0)
    o1 = O.isa_head(Q, K, V, p, gamma=0.3).O
    o2 = O.isa_head(Q, K, V, p, gamma=-0.6).O
    assert np.abs((o2 - o0) + 2.0 * (o1 - o0)).max() < 1e-12
    # the residual is constant over the tokens of a block
    d = o1 - o0
    for s_, n in zip(p.starts, p.counts):
        assert np.abs(d[s_:s_ + n] - d[s_]).max() < 1e-12


def test_coarse_output_is_pooled_sdpa_over_kept_blocks():
    Q, K, V = _rand_head(41, 256, 224, 8)
    p = O.make_plan(256, 224, 32, 0.5, 0.5, 0.25)
    r = O.isa_head(Q, K, V, p)
    J = O.kept_blocks(r.ctx_idx, p)
    ref = _sdpa(r.Qc, r.Kc[J], r.Vc[J])
    assert np.abs(O.coarse_output(r.S, r.Vc, J) - ref).max() < 1e-12


def test_residual_with_unit_blocks_scales_dense_attention():
    # b = 1, all context kept, all sharp: pooling is the identity, so the
    # coarse output is dense attention and O = (1 + gamma) * dense.
    Q, K, V = _rand_head(42, 48, 40, 8)
    p = O.make_plan(48, 40, 1, 1.0, 0.0, 0.5)
    o = O.isa_head(Q, K, V, p, gamma=0.25).O
    assert np.abs(o - 1.25 * _sdpa(Q, K, V)).max() < 1e-12


# --------------------------------------------------------- decoupled RoPE
def _rope64(X, pos, base):
    """Plain fp64 rotary embedding as complex multiplication (no rounding)."""
    D = X.shape[1]
    z = X[:, 0::2] + 1j * X[:, 1::2]
    ang = pos[:, None] * base ** (-(2.0 * np.arange(D // 2)) / D)[None, :]
    r = z * np.exp(1j * ang)
    out = np.empty_like(X)
    out[:, 0::2], out[:, 1::2] = r.real, r.imag
    return out


def test_rope_matches_complex_rotation_and_restarts_per_segment():
    rng = np.random.default_rng(50)
    Ls, Lc, D = 40, 30, 16
    X = isa_inputs.round_to_bf16(rng.standard_normal((Ls + Lc, D)).astype(np.float32))[1]
    pos = O.rope_positions(Ls, Lc)
    assert pos[0] == 0 and pos[Ls] == 0 and pos[-1] == Lc - 1
    R = O.rope(X, Ls, Lc, 10000.0)
    ref = _rope64(X.astype(np.float64), pos, 10000.0)
    assert np.abs(R - ref).max() <= 2 ** -7 * np.abs(ref).max()   # bf16 rounding only
    # identical tokens at equal source/context positions rotate identically
    X2 = X.copy()
    X2[Ls:Ls + 10] = X2[:10]
    R2 = O.rope(X2, Ls, Lc, 10000.0)
    assert np.array_equal(R2[Ls:Ls + 10], R2[:10])
    # position 0 is the identity (bf16 inputs are already representable)
    assert np.array_equal(R[0], X[0].astype(np.float64))


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(51)
    D = 32
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((1, D))
    base = 500.0
    dots = []
    for m, n in ((3, 1), (10, 8), (107, 105)):
        qm = _rope64(q, np.array([m], dtype=np.float64), base)
        kn = _rope64(k, np.array([n], dtype=np.float64), base)
        dots.append(float((qm @ kn.T)[0, 0]))
    assert np.allclose(dots, dots[0], rtol=0, atol=1e-12)
