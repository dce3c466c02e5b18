"""Pins for the oracle's selection margins (the gaps that decide when a
GPU/oracle selection mismatch is excused) and CPU checks of the parity
comparator with planted mismatches. The gaps are hand-computed; each case is
built so that a plausible slip fails it: a reversed sign, an off-by-one
boundary (s[k] - s[k+1] or s[k-2] - s[k-1]), raw instead of normalised
sharpness, or scores taken over all blocks instead of the kept ones."""
import math

import numpy as np
import pytest

import isa_inputs
from oracle import isa_oracle as O
from parity_util import TIE_BAND, compare_head


# ------------------------------------------------------------- _topk_gap
def test_topk_gap_hand_values():
    s = np.array([3.0, 2.0, 2.0, 1.0])
    assert O._topk_gap(s, 1) == 1.0          # 3 kept, best dropped 2
    assert O._topk_gap(s, 2) == 0.0          # exact tie at the boundary
    assert O._topk_gap(s, 3) == 1.0          # 2 kept, 1 dropped
    assert O._topk_gap(s, 0) == math.inf     # nothing kept
    assert O._topk_gap(s, 4) == math.inf     # nothing dropped
    # order of the input does not matter; negative scores
    assert O._topk_gap(np.array([1.0, 2.0, 3.0, 2.0]), 1) == 1.0
    assert O._topk_gap(np.array([-1.0, -5.0, -2.0]), 1) == 1.0
    assert O._topk_gap(np.array([-1.0, -5.0, -2.0]), 2) == 3.0
    # off-by-one and sign slips give other values on this input
    u = np.array([10.0, 7.0, 6.5, 2.0, 1.75])
    assert O._topk_gap(u, 2) == 0.5
    assert O._topk_gap(u, 3) == 4.5


# ------------------------------------------------------------- _split_gap
def _plan8(alpha_f=0.5):
    # 4 source and 4 context blocks of 64 tokens: N_src = 4, N = 8
    return O.make_plan(256, 256, 64, 0.5, alpha_f, 0.5)


def test_split_gap_on_normalised_sharpness():
    p = _plan8()
    assert (p.N_src, p.N, p.n_sharp) == (4, 8, 4)
    norm = np.array([3.0, 0.5, 2.0, 1.25, 0.0, 2.5, 0.25, 1.5])   # N_src^2 * M
    M = norm / p.N_src ** 2
    # sorted: 3.0 2.5 2.0 1.5 | 1.25 0.5 0.25 0 -> 4th kept minus 5th = 0.25
    assert O._split_gap(M, p) == 0.25
    # raw M would give 0.25 / 16; the neighbouring gaps are 0.5 and 0.75
    assert O._split_gap(M, p) != 0.25 / 16
    tie = norm.copy()
    tie[3] = 1.5                                  # 4th and 5th equal
    assert O._split_gap(tie / 16, p) == 0.0
    assert O._split_gap(M, _plan8(0.0)) == math.inf   # every block sharp
    assert O._split_gap(M, _plan8(1.0)) == math.inf   # every block flat


def test_split_gap_matches_one_hot_and_uniform_rows():
    p = _plan8()
    # one-hot softmax row: N_src^2 M = N_src - 1 = 3; uniform row: 0
    M = np.array([3.0, 3.0, 3.0, 3.0, 0.0, 0.0, 0.0, 0.0]) / 16
    assert O._split_gap(M, p) == 3.0


# ------------------------------------------------------------ _exact_gaps
def test_exact_gaps_over_kept_blocks_only():
    p = O.make_plan(256, 256, 64, 0.5, 0.5, 0.5)   # N_kv = 6, k_ns = 3
    assert (p.N_kv, p.k_ns) == (6, 3)
    J = np.array([0, 1, 2, 3, 5, 7])
    S = np.full((p.N, p.N), 5.0)                    # pruned columns 4, 6 score 5.0
    S[2, J] = [0.9, 0.1, 0.5, 0.3, 0.7, 0.2]        # top 3: .9 .7 .5, 4th .3
    S[6, J] = [0.4, 0.4, 0.4, 0.4, 0.1, 0.0]        # tie at the boundary
    g = O._exact_gaps(S, J, np.array([6, 2]), p)
    assert g.shape == (2,)
    assert g[0] == 0.0
    assert abs(g[1] - 0.2) < 1e-15


def test_head_result_reports_the_helpers_gaps():
    """isa_head's reported gaps are the helpers' values on its own scores."""
    p = O.make_plan(700, 451, 64, 0.25, 0.5, 0.125)
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((1151, 64)) for _ in range(3))
    r = O.isa_head(Q, K, V, p, compute_output=False)
    J = O.kept_blocks(r.ctx_idx, p)
    assert r.split_gap == O._split_gap(r.sharpness, p)
    assert np.array_equal(r.exact_gaps, O._exact_gaps(r.S, J, r.flat_idx, p))
    assert r.ctx_gap == O._topk_gap(r.ctx_score, p.k_ctx)
    assert r.split_gap > TIE_BAND and r.ctx_gap > TIE_BAND


# ------------------------------------------------------ comparator checks
def _fake_gpu(r, plan, O_rows=None):
    return {"ctx_idx": r.ctx_idx + plan.N_src, "sharp_idx": r.sharp_idx.copy(),
            "flat_idx": r.flat_idx.copy(), "flat_exact_idx": r.flat_exact_idx.copy(),
            "O": (r.O if O_rows is None else O_rows).copy()}


def _head(seed=5, L_src=700, L_ctx=451, D=32, b=64, a_s=0.25, a_f=0.5, a_ns=0.25):
    """One head of the clustered generator (fp64 copies, edited in place by
    the tests that plant ties)."""
    p = O.make_plan(L_src, L_ctx, b, a_s, a_f, a_ns)
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in isa_inputs.make_head(50 + seed, 0, 0, L_src, L_ctx, D))
    return p, Q, K, V


def test_comparator_equal_selections_compare_every_row():
    p, Q, K, V = _head()
    r = O.isa_head(Q, K, V, p)
    rep = compare_head(p, Q, K, V, _fake_gpu(r, p), oracle_result=r)
    assert rep["excused"] == [] and rep["n_compared"] == Q.size and rep["n_rows_skipped"] == 0


def test_comparator_rejects_selection_outside_the_band():
    p, Q, K, V = _head()
    r = O.isa_head(Q, K, V, p)
    g = _fake_gpu(r, p)
    g["sharp_idx"][0], g["flat_idx"][0] = g["flat_idx"][0], g["sharp_idx"][0]
    g["sharp_idx"].sort(), g["flat_idx"].sort()
    with pytest.raises(AssertionError, match="split differs"):
        compare_head(p, Q, K, V, g, oracle_result=r)
    g = _fake_gpu(r, p)
    g["flat_exact_idx"][0, 0] = O.kept_blocks(r.ctx_idx, p)[-1] if r.flat_exact_idx[0, 0] != \
        O.kept_blocks(r.ctx_idx, p)[-1] else O.kept_blocks(r.ctx_idx, p)[-2]
    g["flat_exact_idx"][0].sort()
    with pytest.raises(AssertionError, match="exact set"):
        compare_head(p, Q, K, V, g, oracle_result=r)
    g = _fake_gpu(r, p)
    g["O"][5, 3] += 0.05
    with pytest.raises(AssertionError):
        compare_head(p, Q, K, V, g, oracle_result=r)


def test_comparator_split_tie_skips_only_the_swapped_blocks():
    """Two query blocks with identical tokens have identical sharpness; when
    they sit on the sharp/flat boundary either may be sharp. The rows of the
    two swapped blocks are left out, every other row is still compared, and
    the exact sets of the other flat blocks are still checked."""
    p, Q, K, V = _head(seed=8)
    r0 = O.isa_head(Q, K, V, p, compute_output=False)
    order = np.lexsort((np.arange(p.N), -r0.sharpness))
    a, c = int(order[p.n_sharp - 1]), int(order[p.n_sharp])   # last sharp, first flat
    sa, sc = p.starts[a], p.starts[c]
    assert p.counts[a] == p.counts[c] == 64
    Q[sc:sc + 64] = Q[sa:sa + 64]                     # block c now scores exactly like block a
    r = O.isa_head(Q, K, V, p)
    assert r.split_gap == 0.0
    lo, hi = min(a, c), max(a, c)
    assert lo in r.sharp_idx and hi in r.flat_idx      # ties: the lower index is sharper
    g = _fake_gpu(r, p)
    g["sharp_idx"] = np.sort(np.where(r.sharp_idx == lo, hi, r.sharp_idx))
    g["flat_idx"] = np.sort(np.where(r.flat_idx == hi, lo, r.flat_idx))
    # the GPU's exact set for its flat block `lo` (its scores equal those of `hi`)
    rows_E = {int(i): e for i, e in zip(r.flat_idx, r.flat_exact_idx)}
    rows_E[lo] = rows_E.pop(hi)
    g["flat_exact_idx"] = np.stack([rows_E[int(i)] for i in g["flat_idx"]])
    rep = compare_head(p, Q, K, V, g, oracle_result=r)
    assert [e[0] for e in rep["excused"]] == ["split"]
    assert rep["n_rows_skipped"] == 128
    assert rep["n_compared"] == (Q.shape[0] - 128) * Q.shape[1]
    # an exact set of another flat block is still compared
    g2 = {k: v.copy() for k, v in g.items()}
    k = next(k for k, i in enumerate(g2["flat_idx"]) if i not in (lo, hi))
    J = O.kept_blocks(r.ctx_idx, p)
    other = next(j for j in J if j not in g2["flat_exact_idx"][k])
    g2["flat_exact_idx"][k, 0] = other
    g2["flat_exact_idx"][k].sort()
    with pytest.raises(AssertionError, match="exact set"):
        compare_head(p, Q, K, V, g2, oracle_result=r)


def test_comparator_context_tie_compares_no_row_but_checks_the_split():
    """Two context blocks with identical keys tie in the context score; a GPU
    keeping the other one is excused, no output row has a unique value, and
    the split (which reads the source columns only) is still checked."""
    p, Q, K, V = _head(seed=9, a_s=0.5)
    r0 = O.isa_head(Q, K, V, p, compute_output=False)
    order = np.lexsort((np.arange(p.N_ctx), -r0.ctx_score))
    kept, dropped = int(order[p.k_ctx - 1]), int(order[p.k_ctx])
    sk, sd = p.starts[p.N_src + kept], p.starts[p.N_src + dropped]
    assert p.counts[p.N_src + kept] == p.counts[p.N_src + dropped] == 64
    K[sd:sd + 64] = K[sk:sk + 64]
    r = O.isa_head(Q, K, V, p)
    assert r.ctx_gap == 0.0
    lo, hi = min(kept, dropped), max(kept, dropped)
    g = _fake_gpu(r, p)
    g["ctx_idx"] = np.sort(np.where(r.ctx_idx == lo, hi, r.ctx_idx)) + p.N_src
    rep = compare_head(p, Q, K, V, g, oracle_result=r)
    assert [e[0] for e in rep["excused"]] == ["ctx"]
    assert rep["n_compared"] == 0 and rep["n_rows_skipped"] == Q.shape[0]
    g["sharp_idx"][0], g["flat_idx"][0] = g["flat_idx"][0], g["sharp_idx"][0]
    g["sharp_idx"].sort(), g["flat_idx"].sort()
    with pytest.raises(AssertionError, match="split differs"):
        compare_head(p, Q, K, V, g, oracle_result=r)


def test_oracle_pool_checks_regenerated_heads():
    """The worker processes of the GPU tests regenerate a head from its seed
    and run the comparator: a copy of the oracle's own results passes, a
    planted output error is reported from the worker."""
    from parity_util import OraclePool, head_values
    stream, Ls, Lc, D, b, ratios = 1, 300, 200, 64, 64, (0.25, 0.5, 0.25)
    plan = O.make_plan(Ls, Lc, b, *ratios)
    jobs = []
    for h in range(2):
        Qv, Kv, Vv = head_values(stream, 0, h, Ls, Lc, D)
        r = O.isa_head(Qv, Kv, Vv, plan)
        gpu = _fake_gpu(r, plan)
        if h == 1:
            rows = np.array([0, 5, Ls, Ls + Lc - 1])
            gpu["O_rows"] = gpu.pop("O")[rows]
        else:
            rows = None
        jobs.append(dict(stream=stream, bi=0, h=h, L_src=Ls, L_ctx=Lc, D=D, b=b, ratios=ratios,
                         gpu=gpu, rows=rows))
    with OraclePool() as pool:
        reps = pool.run(jobs)
        assert reps[0]["n_compared"] == (Ls + Lc) * D and reps[1]["n_compared"] == 4 * D
        bad = dict(jobs[1], gpu=dict(jobs[1]["gpu"], O_rows=jobs[1]["gpu"]["O_rows"] + 0.1))
        with pytest.raises(AssertionError):
            pool.run([bad])
