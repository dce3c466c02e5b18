"""Comparison of the HIP path against the CPU oracle (test infrastructure).

Selections (kept context blocks, sharp/flat split, exact sets E_i) must be
identical as ascending id lists. A mismatch is excused only where the
oracle's own score gap at the selection boundary is below TIE_BAND: for a
top-k the gap is the k-th kept score minus the best dropped score; for the
split it is measured on the normalised sharpness N_src^2 * M_i. An excused
selection must still be a valid choice under the oracle's scores (every
chosen score within TIE_BAND of the oracle's boundary). The oracle never
takes a selection from the GPU: the rows whose value depends on an excused
choice have no unique expected value and are left out of the comparison,
and only those rows:
  * a different context selection changes J, which every row attends over:
    no row is compared (the split is still checked, since sharpness reads
    the source columns only);
  * a different split leaves out the rows of the blocks whose path differs;
    the exact sets of blocks flat on both sides are still compared;
  * a different exact set leaves out the rows of that flat block.
All other requested rows must agree within MAX_ABS / MEAN_ABS.
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


def _block_rows(plan, i):
    s0 = plan.starts[i]
    return slice(s0, s0 + plan.counts[i])


def compare_head(plan, Qv, Kv, Vv, gpu, rows=None, oracle_result=None):
    """gpu: dict of numpy arrays for one (batch, head): ctx_idx (global ids),
    sharp_idx, flat_idx, flat_exact_idx, and either O ([L, D] float) or
    O_rows (the rows listed in `rows`, in that order). rows: token rows to
    compare (None = all). Returns a report dict (n_compared = output
    elements compared, n_rows_skipped = requested rows left out because an
    excused selection leaves them no unique value); raises AssertionError on
    a parity failure."""
    r = oracle_result or isa_oracle.isa_head(Qv, Kv, Vv, plan, rows=rows)
    L = Qv.shape[0]
    rep = {"excused": [], "oracle": r, "max_abs": 0.0, "mean_abs": 0.0, "rel_l2": 0.0,
           "n_compared": 0, "n_rows_skipped": 0}
    skip = np.zeros(L, dtype=bool)

    # step (2): kept context blocks
    g_ctx = np.asarray(gpu["ctx_idx"], dtype=np.int64) - plan.N_src
    ctx_same = np.array_equal(g_ctx, r.ctx_idx)
    if not ctx_same:
        assert r.ctx_gap < TIE_BAND, f"ctx top-k differs (oracle gap {r.ctx_gap:.3e})"
        assert _valid_choice(r.ctx_score, g_ctx, plan.k_ctx), "ctx top-k is not a valid choice"
        assert np.all(np.diff(g_ctx) > 0), "ctx list not ascending"
        rep["excused"].append(("ctx", float(r.ctx_gap)))
        skip[:] = True

    # step (3): the split (independent of J)
    g_sh = np.asarray(gpu["sharp_idx"], dtype=np.int64)
    g_fl = np.asarray(gpu["flat_idx"], dtype=np.int64)
    assert g_sh.size == plan.n_sharp and g_fl.size == plan.n_flat, "split sizes"
    assert np.array_equal(np.sort(np.concatenate([g_sh, g_fl])), np.arange(plan.N)), "split is not a partition"
    assert np.all(np.diff(g_sh) > 0) and np.all(np.diff(g_fl) > 0), "split lists not ascending"
    if not np.array_equal(g_sh, r.sharp_idx):
        assert r.split_gap < TIE_BAND, f"sharp/flat split differs (oracle gap {r.split_gap:.3e})"
        assert _valid_choice(r.sharpness * plan.N_src ** 2, g_sh, plan.n_sharp), "split is not valid"
        rep["excused"].append(("split", float(r.split_gap)))
        for i in np.setxor1d(g_sh, r.sharp_idx):      # blocks whose path differs
            skip[_block_rows(plan, int(i))] = True

    # step (5): exact sets of the blocks flat on both sides
    if ctx_same and plan.n_flat and plan.k_ns:
        J = isa_oracle.kept_blocks(r.ctx_idx, plan)
        o_row = {int(i): k for k, i in enumerate(r.flat_idx)}
        g_E = np.asarray(gpu["flat_exact_idx"], dtype=np.int64).reshape(plan.n_flat, plan.k_ns)
        for k, i in enumerate(g_fl):
            ko = o_row.get(int(i))
            if ko is None or np.array_equal(g_E[k], r.flat_exact_idx[ko]):
                continue
            gap = float(r.exact_gaps[ko])
            assert gap < TIE_BAND, f"exact set of flat block {i} differs (oracle gap {gap:.3e})"
            pos = np.searchsorted(J, g_E[k])
            assert np.all(pos < J.size) and np.array_equal(J[np.minimum(pos, J.size - 1)], g_E[k]), \
                "exact set outside J"
            assert _valid_choice(r.S[i, J], pos, plan.k_ns), "exact set is not a valid choice"
            rep["excused"].append(("exact", gap))
            skip[_block_rows(plan, int(i))] = True

    want = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    keep = ~skip[want]
    rep["n_rows_skipped"] = int((~keep).sum())
    if not keep.any():
        return rep
    ref = r.O[want[keep]]
    assert np.isfinite(ref).all(), "oracle rows missing"
    if "O" in gpu:
        got = np.asarray(gpu["O"], dtype=np.float64)[want[keep]]
    else:   # only the requested rows, in the order of `rows`
        got = np.asarray(gpu["O_rows"], dtype=np.float64)[keep]
    assert np.isfinite(got).all(), "non-finite GPU output"
    err = np.abs(got - ref)
    rep.update(max_abs=float(err.max()), mean_abs=float(err.mean()),
               rel_l2=float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)),
               n_compared=int(err.size))
    assert rep["max_abs"] <= MAX_ABS and rep["mean_abs"] <= MEAN_ABS, {
        k: v for k, v in rep.items() if k != "oracle"}
    return rep


# ------------------------------------------------ oracle heads in parallel
# The GPU tests compare many heads; the oracle runs them in worker processes
# started fresh (spawn: no GPU state is inherited, and workers import numpy
# and the oracle only). Each worker regenerates its head from the seeded
# generator, so only the GPU's results travel to it.
ORACLE_WORKERS = 4          # x ORACLE_THREADS BLAS threads: 16 host cores
ORACLE_THREADS = 4


def _worker_init(threads):
    try:
        from threadpoolctl import threadpool_limits
        globals()["_blas_limit"] = threadpool_limits(threads)
    except ImportError:
        pass


def head_values(stream, bi, h, L_src, L_ctx, D):
    """The bf16 values (as fp32) of one generated head: what the GPU received."""
    import isa_inputs
    return tuple(isa_inputs.round_to_bf16(x)[1] for x in isa_inputs.make_head(stream, bi, h, L_src, L_ctx, D))


def check_head_job(job):
    """Worker: the oracle on one generated head against the GPU's results.
    job: dict(stream, bi, h, L_src, L_ctx, D, b, ratios=(a_s, a_f, a_ns),
    gpu=..., rows=None | array). Returns compare_head's report without the
    oracle's arrays (AssertionError on a parity failure)."""
    plan = isa_oracle.make_plan(job["L_src"], job["L_ctx"], job["b"], *job["ratios"])
    Qv, Kv, Vv = head_values(job["stream"], job["bi"], job["h"], job["L_src"], job["L_ctx"], job["D"])
    rep = compare_head(plan, Qv, Kv, Vv, job["gpu"], rows=job["rows"])
    rep.pop("oracle")
    rep["head"] = (job["bi"], job["h"])
    return rep


class OraclePool:
    """Process pool for check_head_job (context manager)."""

    def __enter__(self):
        import concurrent.futures as cf
        import multiprocessing as mp
        self.ex = cf.ProcessPoolExecutor(max_workers=ORACLE_WORKERS, mp_context=mp.get_context("spawn"),
                                         initializer=_worker_init, initargs=(ORACLE_THREADS,))
        return self

    def run(self, jobs):
        """Reports in the order of `jobs`; the first failure is raised."""
        futs = [self.ex.submit(check_head_job, j) for j in jobs]
        return [f.result() for f in futs]

    def __exit__(self, *exc):
        self.ex.shutdown(wait=True, cancel_futures=True)
        return False
