"""Comparison of the HIP path against the CPU oracle (test infrastructure).

Selections (kept context blocks, sharp/flat split, exact sets E_i) must be
identical as ascending id lists. A mismatch is excused only where the
oracle's own score gap at the selection boundary is below TIE_BAND: for a
top-k the gap is the k-th kept score minus the best dropped score; for the
split it is measured on the normalised sharpness N_src^2 * M_i. Excused
selections are injected into the oracle, which then recomputes the outputs.
Outputs must agree within MAX_ABS / MEAN_ABS over every compared element.
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


def compare_head(plan, Qv, Kv, Vv, gpu, rows=None, oracle_result=None):
    """gpu: dict of numpy arrays for one (batch, head): ctx_idx (global ids),
    sharp_idx, flat_idx, flat_exact_idx, O ([L, D] float). rows: token rows
    to compare (None = all). Returns a report dict; raises AssertionError on
    a parity failure."""
    r = oracle_result or isa_oracle.isa_head(Qv, Kv, Vv, plan, rows=rows)
    rep = {"excused": []}
    g_ctx = np.asarray(gpu["ctx_idx"], dtype=np.int64) - plan.N_src
    inject = {}
    if not np.array_equal(g_ctx, r.ctx_idx):
        assert r.ctx_gap < TIE_BAND, f"ctx top-k differs (oracle gap {r.ctx_gap:.3e})"
        rep["excused"].append(("ctx", r.ctx_gap))
        inject["ctx_idx"] = g_ctx
    g_sh = np.asarray(gpu["sharp_idx"], dtype=np.int64)
    g_fl = np.asarray(gpu["flat_idx"], dtype=np.int64)
    if inject:
        r = isa_oracle.isa_head(Qv, Kv, Vv, plan, selections=dict(inject), rows=rows)
    if not (np.array_equal(g_sh, r.sharp_idx) and np.array_equal(g_fl, r.flat_idx)):
        assert r.split_gap < TIE_BAND, f"sharp/flat split differs (oracle gap {r.split_gap:.3e})"
        rep["excused"].append(("split", r.split_gap))
        inject.update(sharp_idx=g_sh, flat_idx=g_fl)
        r = isa_oracle.isa_head(Qv, Kv, Vv, plan, selections=dict(inject), rows=rows)
    g_E = np.asarray(gpu["flat_exact_idx"], dtype=np.int64).reshape(len(g_fl), plan.k_ns)
    bad_rows = [i for i in range(len(g_fl)) if not np.array_equal(g_E[i], r.flat_exact_idx[i])]
    for i in bad_rows:
        assert r.exact_gaps[i] < TIE_BAND, (
            f"exact set of flat block {g_fl[i]} differs (oracle gap {r.exact_gaps[i]:.3e})")
        rep["excused"].append(("exact", float(r.exact_gaps[i])))
    if bad_rows:
        inject["flat_exact_idx"] = g_E
        r = isa_oracle.isa_head(Qv, Kv, Vv, plan, selections=dict(inject), rows=rows)
    want = np.arange(Qv.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    rep["oracle"] = r
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
