"""Comparison of the HIP path against the CPU oracle (test infrastructure).

Selections (kept context blocks, sharp/flat split, exact sets E_i) must be
identical as ascending id lists. A mismatch is excused only where the
oracle's own score gap at the selection boundary is below TIE_BAND: for a
top-k the gap is the k-th kept score minus the best dropped score; for the
split it is measured on the normalised sharpness N_src^2 * M_i. An excused
selection must still be a valid choice under the oracle's scores (every
chosen score within TIE_BAND of the oracle's boundary); the outputs that
depend on it have no unique value and are not compared (the whole head for
the context or split selection, the rows of that flat block for an E_i).
The oracle only ever runs on the generated inputs. All other outputs must
agree within MAX_ABS / MEAN_ABS over every compared element.
"""
from __future__ import annotations

import numpy as np

from oracle import isa_oracle

TIE_BAND = 1e-5
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def bf16_tensor(bits, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def _valid_choice(scores, chosen, k):
    """`chosen` is a valid top-k of `scores` up to ties: k distinct ids whose
    scores all reach the oracle's k-th largest score minus TIE_BAND."""
    chosen = np.asarray(chosen, dtype=np.int64)
    kth = np.sort(np.asarray(scores, dtype=np.float64))[::-1][k - 1]
    return (chosen.size == k and np.unique(chosen).size == k
            and bool((np.asarray(scores)[chosen] >= kth - TIE_BAND).all()))


def compare_head(plan, Qv, Kv, Vv, gpu, rows=None, oracle_result=None):
    """gpu: dict of numpy arrays for one (batch, head): ctx_idx (global ids),
    sharp_idx, flat_idx, flat_exact_idx, O ([L, D] float). rows: token rows
    to compare (None = all). Returns a report dict; raises AssertionError on
    a parity failure."""
    r = oracle_result or isa_oracle.isa_head(Qv, Kv, Vv, plan, rows=rows)
    rep = {"excused": [], "oracle": r, "max_abs": 0.0, "mean_abs": 0.0, "rel_l2": 0.0, "n_compared": 0}
    g_ctx = np.asarray(gpu["ctx_idx"], dtype=np.int64) - plan.N_src
    if not np.array_equal(g_ctx, r.ctx_idx):
        assert r.ctx_gap < TIE_BAND, f"ctx top-k differs (oracle gap {r.ctx_gap:.3e})"
        assert _valid_choice(r.ctx_score, g_ctx, plan.k_ctx), "ctx top-k is not a valid choice"
        rep["excused"].append(("ctx", r.ctx_gap))
        return rep
    g_sh = np.asarray(gpu["sharp_idx"], dtype=np.int64)
    g_fl = np.asarray(gpu["flat_idx"], dtype=np.int64)
    if not (np.array_equal(g_sh, r.sharp_idx) and np.array_equal(g_fl, r.flat_idx)):
        assert r.split_gap < TIE_BAND, f"sharp/flat split differs (oracle gap {r.split_gap:.3e})"
        assert _valid_choice(r.sharpness * plan.N_src ** 2, g_sh, plan.n_sharp), "split is not valid"
        assert np.array_equal(np.sort(np.concatenate([g_sh, g_fl])), np.arange(plan.N))
        rep["excused"].append(("split", r.split_gap))
        return rep
    g_E = np.asarray(gpu["flat_exact_idx"], dtype=np.int64).reshape(len(g_fl), plan.k_ns)
    J = isa_oracle.kept_blocks(r.ctx_idx, plan)
    skip = np.zeros(Qv.shape[0], dtype=bool)
    for i in range(len(g_fl)):
        if np.array_equal(g_E[i], r.flat_exact_idx[i]):
            continue
        assert r.exact_gaps[i] < TIE_BAND, (
            f"exact set of flat block {g_fl[i]} differs (oracle gap {r.exact_gaps[i]:.3e})")
        pos = np.searchsorted(J, g_E[i])
        assert np.array_equal(J[pos], g_E[i]), "exact set outside J"
        assert _valid_choice(r.S[g_fl[i], J], pos, plan.k_ns), "exact set is not a valid choice"
        rep["excused"].append(("exact", float(r.exact_gaps[i])))
        s0 = plan.starts[g_fl[i]]
        skip[s0:s0 + plan.counts[g_fl[i]]] = True
    want = np.arange(Qv.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    want = want[~skip[want]]
    if want.size == 0:
        return rep
    ref = r.O[want]
    got = np.asarray(gpu["O"], dtype=np.float64)[want]
    assert np.isfinite(got).all(), "non-finite GPU output"
    err = np.abs(got - ref)
    rep.update(max_abs=float(err.max()), mean_abs=float(err.mean()),
               rel_l2=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)),
               n_compared=int(err.size))
    assert rep["max_abs"] <= MAX_ABS and rep["mean_abs"] <= MEAN_ABS, {
        k: v for k, v in rep.items() if k != "oracle"}
    return rep
