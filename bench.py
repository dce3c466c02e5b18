"""Benchmark of the ISA forward pass on one MI355X.

Workload: In-context Sparse Attention forward at 64K tokens
(B=1, H=40, D=128, L_src = L_ctx = 32768, b=64, alpha_s=0.125, alpha_f=0.5,
alpha_ns=0.0625), bf16 inputs from the seeded clustered generator, resident in
HBM before timing starts.

One step = one pass of the whole hot path through the C ABI: pooling,
context top-k, coarse rows + sharpness + split + exact sets, sharp attention,
flat exact+Taylor attention. The step is issued as the five entry points on
torch's current stream with HIP events between them (per-kernel durations
for the roofline); the isa_forward entry point (same kernels in one call) is
timed as well, as is the library's dense attention on the same inputs, and,
for context, PyTorch's flash scaled_dot_product_attention on them.

Prints one JSON line. `value` is the forward latency in ms (lower is better).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ISA fwd latency (ms) + effective TFLOP/s & MFMA util at 64K tokens, H=40, D=128"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6     # dense fp64 matrix-core peak
WORKLOAD = dict(stream=4, B=1, H=40, L_src=32768, L_ctx=32768, D=128, b=64,
                alpha_s=0.125, alpha_f=0.5, alpha_ns=0.0625)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sharp_attn_64k_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_attention_blockwise_amd", "csrc", "isa_attn.hip")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["sharp"], default=None,
                    help="launch only this kernel --steps times (for counter collection)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="131072-token grid of (b, alpha_s, alpha_ns, alpha_f) against dense attention")
    ap.add_argument("--backward", action="store_true",
                    help="time isa_forward + isa_backward (and the dense configuration on the same kernels)")
    ap.add_argument("--fig6", action="store_true",
                    help="pure 0th-order Taylor variant (alpha_f=1, alpha_ns=0) vs exact "
                         "attention over J: latencies and the error/sharpness rank correlation")
    return ap.parse_args()


def make_inputs(dev):
    import torch
    import isa_inputs
    w = WORKLOAD
    L = w["L_src"] + w["L_ctx"]
    shape = (w["B"], w["H"], L, w["D"])
    out = {n: torch.empty(shape, dtype=torch.bfloat16, device=dev) for n in "QKV"}
    host = {}
    for bi in range(w["B"]):
        for h in range(w["H"]):
            qkv = isa_inputs.make_head(w["stream"], bi, h, w["L_src"], w["L_ctx"], w["D"])
            for n, x in zip("QKV", qkv):
                bits, val = isa_inputs.round_to_bf16(x)
                out[n][bi, h].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
                if (bi, h) == (0, 0):
                    host[n] = val
    return out, host


def block_counts(p, pl):
    """Valid tokens n_j of every global block, by the library's block-cut rule
    (each segment cut on its own; a tail block holds the remainder)."""
    src = [min(p.b, p.L_src - j * p.b) for j in range(pl["N_src"])]
    ctx = [min(p.b, p.L_ctx - j * p.b) for j in range(pl["N_ctx"])]
    return np.asarray(src + ctx, dtype=np.float64)


def block_starts(p, pl):
    return np.asarray([j * p.b for j in range(pl["N_src"])] +
                      [p.L_src + j * p.b for j in range(pl["N_ctx"])], dtype=np.int64)


def algorithmic_flops(p, pl, ctx_idx, sharp_idx, flat_idx, exact_idx):
    """FLOPs of the method from the actual selections (4*D per query-key pair
    for the exact terms and the pooled terms, 2*D per coarse score)."""
    n = block_counts(p, pl)
    D = p.D
    f_sharp = f_flat = f_taylor = 0.0
    for bi in range(p.B):
        for h in range(p.H):
            J = np.concatenate([np.arange(pl["N_src"]), ctx_idx[bi, h]])
            nJ = n[J].sum()
            f_sharp += 4 * D * n[sharp_idx[bi, h]].sum() * nJ
            fi = flat_idx[bi, h]
            if fi.size:
                nE = n[exact_idx[bi, h]].sum(axis=1)
                f_flat += 4 * D * (n[fi] * nE).sum()
                f_taylor += 4 * D * (n[fi] * (pl["N_kv"] - pl["k_ns"])).sum()
    f_coarse = 2 * D * pl["N"] * pl["N_kv"] * p.B * p.H
    L = p.L_src + p.L_ctx
    f_dense = 4 * D * L * L * p.B * p.H
    return dict(sharp=f_sharp, flat_exact=f_flat, taylor=f_taylor, coarse=f_coarse, dense=f_dense)


def traffic_record():
    """HBM bytes per launch of the sharp kernel from the committed rocprofv3
    counter summary, valid only for the kernel source it was taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """Cores this process may run on and the CPU model name."""
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(host, budget_s):
    """The CPU oracle, untuned, on a bounded sample of the same workload:
    head (0,0) with its selections in full and outputs for as many sharp and
    flat query blocks as fit the time budget, extrapolated to the whole
    forward (all blocks, all heads)."""
    from oracle import isa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = WORKLOAD
    plan = O.make_plan(w["L_src"], w["L_ctx"], w["b"], w["alpha_s"], w["alpha_f"], w["alpha_ns"])
    Q, K, V = (host[n].astype(np.float64) for n in "QKV")
    t0 = time.perf_counter()
    sel = O.isa_head(Q, K, V, plan, compute_output=False)
    t_sel = time.perf_counter() - t0
    sel_d = dict(ctx_idx=sel.ctx_idx, sharp_idx=sel.sharp_idx, flat_idx=sel.flat_idx,
                 flat_exact_idx=sel.flat_exact_idx)
    rng = np.random.default_rng(0)
    sharp_order = rng.permutation(sel.sharp_idx)
    flat_order = rng.permutation(sel.flat_idx)
    # Each oracle call with injected selections repeats the head's pooling
    # and coarse steps; G blocks per call spread that fixed part, and its
    # own time (the median of a few calls with no rows) is taken off.
    G = 8
    t_fixed = []
    for _ in range(3):
        t1 = time.perf_counter()
        O.isa_head(Q, K, V, plan, selections=sel_d, rows=np.zeros(0, dtype=np.int64))
        t_fixed.append(time.perf_counter() - t1)
    t_fixed = float(np.median(t_fixed))
    done = {"sharp": [], "flat": []}
    per_call = {"sharp": [], "flat": []}
    deadline = time.perf_counter() + budget_s
    k = 0
    while time.perf_counter() < deadline or min(len(per_call["sharp"]), len(per_call["flat"])) < 2:
        for kind, order in (("sharp", sharp_order), ("flat", flat_order)):
            blocks = order[k:k + G]
            if len(blocks) == 0:
                continue
            rows = np.concatenate([np.arange(plan.starts[i], plan.starts[i] + plan.counts[i]) for i in blocks])
            t1 = time.perf_counter()
            O.isa_head(Q, K, V, plan, selections=sel_d, rows=rows)
            per_call[kind].append((time.perf_counter() - t1 - t_fixed) / len(blocks))
            done[kind].extend(blocks)
        k += G
        if k >= max(len(sharp_order), len(flat_order)):
            break
    per_sharp = max(float(np.median(per_call["sharp"])), 0.0) if per_call["sharp"] else 0.0
    per_flat = max(float(np.median(per_call["flat"])), 0.0) if per_call["flat"] else 0.0
    per_head = t_sel + per_sharp * plan.n_sharp + per_flat * plan.n_flat
    total_ms = per_head * w["B"] * w["H"] * 1e3
    host_cores, model = host_cpu()
    return {"value": total_ms, "unit": "ms", "cores": int(threads), "host_cores": host_cores,
            "cpu_model": model, "kind": "oracle",
            "sample": (f"head (0,0) of {w['B'] * w['H']}: selections in full ({t_sel:.2f} s), outputs of "
                       f"{len(done['sharp'])} sharp and {len(done['flat'])} flat query blocks "
                       f"(of {plan.n_sharp}/{plan.n_flat}), {G} per oracle call less the call's fixed "
                       f"part ({t_fixed:.3f} s); median per-block times extrapolated to all "
                       f"blocks and heads, numpy fp64 with {threads} BLAS threads")}


def fig6(isa, torch, p, Q, K, V, args):
    """Sharpness as an error predictor (Fig. 6 of the paper) and the speed of
    the all-Taylor variant (Fig. 8), on the GPU at the benchmark workload.
    Exact reference: alpha_f = 0 (every block exact over J). Taylor variant:
    alpha_f = 1, alpha_ns = 0 (every block on the pooled keys only)."""
    import dataclasses
    from scipy.stats import spearmanr
    pe = dataclasses.replace(p, alpha_f=0.0)
    pt = dataclasses.replace(p, alpha_f=1.0, alpha_ns=0.0)
    times = {}
    outs = {}
    for name, q in (("default", p), ("exact_over_J", pe), ("all_taylor", pt)):
        O, dbg = isa.forward(Q, K, V, q, debug=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(max(args.steps // 4, 2)):
            isa.forward(Q, K, V, q, out=O)
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / max(args.steps // 4, 2)
        outs[name] = (O.float(), dbg["sharpness"])
    pl = isa.plan(p)
    counts = torch.tensor(block_counts(p, pl).astype(np.int64), device=Q.device)
    tok_block = torch.repeat_interleave(torch.arange(pl["N"], device=Q.device), counts)
    diff = (outs["all_taylor"][0] - outs["exact_over_J"][0]).abs().mean(dim=-1)   # [B,H,L]
    rhos = []
    for bi in range(p.B):
        for h in range(p.H):
            err = torch.zeros(pl["N"], device=Q.device, dtype=torch.float32)
            err.index_add_(0, tok_block, diff[bi, h])
            err = (err / counts).cpu().numpy()
            rhos.append(spearmanr(outs["all_taylor"][1][bi, h].cpu().numpy(), err).correlation)
    rhos = np.asarray(rhos)
    print(json.dumps({"fig6": {"spearman_sharpness_vs_taylor_error": {
        "mean": float(rhos.mean()), "min": float(rhos.min()), "max": float(rhos.max()),
        "heads": int(rhos.size)},
        "latency_ms": times,
        "speedup_vs_exact_over_J": {"default": times["exact_over_J"] / times["default"],
                                    "all_taylor": times["exact_over_J"] / times["all_taylor"]},
        "config": {"workload": "isa_fwd_64k_tokens_h40_d128", "alpha_s": p.alpha_s}}}), flush=True)


def backward_bench(isa, torch, p, Q, K, V, args):
    """Training step of the operator (isa_forward + isa_backward) at the
    benchmark workload, and the same kernels in the dense configuration
    (alpha_s = 1, alpha_f = 0: every block exact over every token), which is
    the dense attention forward + backward on this engine."""
    import dataclasses
    pd = dataclasses.replace(p, alpha_s=1.0, alpha_f=0.0)
    g = torch.Generator(device=Q.device).manual_seed(5)
    dO = torch.randn(Q.shape, device=Q.device, generator=g).to(torch.bfloat16)
    res = {}
    runs = [("isa", p)] + ([] if args.no_dense else [("dense_same_engine", pd)])
    for name, q in runs:
        ws = isa.workspace(q, Q.device)
        O = isa.forward(Q, K, V, q, workspace=ws)
        grads = isa.backward(Q, K, V, O, dO, q, ws)
        torch.cuda.synchronize()
        reps = max(args.steps // 4, 2) if name == "isa" else max(args.dense_reps, 1)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        fwd = bwd = 0.0
        for _ in range(reps):
            ev[0].record()
            isa.forward(Q, K, V, q, out=O, workspace=ws)
            ev[1].record()
            isa.backward(Q, K, V, O, dO, q, ws, out=grads)
            ev[2].record()
            torch.cuda.synchronize()
            fwd += ev[0].elapsed_time(ev[1])
            bwd += ev[1].elapsed_time(ev[2])
        res[name] = {"forward_ms": fwd / reps, "backward_ms": bwd / reps,
                     "step_ms": (fwd + bwd) / reps}
        del ws, grads
    if not args.no_dense:
        L = p.L_src + p.L_ctx
        dense_bwd_flop = 10 * p.D * L * L * p.B * p.H   # 5 products of 2*D per query-key pair
        res["dense_same_engine"]["backward_tflops_algorithmic"] = (
            dense_bwd_flop / (res["dense_same_engine"]["backward_ms"] * 1e-3) / 1e12)
        res["speedup_vs_dense_same_engine"] = {
            "backward": res["dense_same_engine"]["backward_ms"] / res["isa"]["backward_ms"],
            "forward_plus_backward": res["dense_same_engine"]["step_ms"] / res["isa"]["step_ms"]}
    print(json.dumps({"backward": res, "config": {"workload": "isa_fwd_64k_tokens_h40_d128"}}),
          flush=True)


# Algorithmic HBM bytes per launch of the selection kernels and pooling
# (B*H heads): what each kernel must read and write once, nothing re-read.
def selection_bytes(p, pl):
    BH, D, N = p.B * p.H, p.D, pl["N"]
    L = p.L_src + p.L_ctx
    return {
        "pool_kernel": 3 * BH * L * D * 2 + BH * N * D * (8 + 8 + 2 + 2),
        "ctx_topk_kernel": BH * ((pl["N_src"] + pl["N_ctx"]) * D * 8 + pl["k_ctx"] * 4 + pl["N_ctx"] * 8),
        "sharpness_kernel": BH * ((N + pl["N_src"]) * D * 8 + N * 8),
        "split_kernel": BH * N * (8 + 4),
        # LDS-row and persistent global-row forms share this prefix
        "flat_topk_": BH * ((pl["n_flat"] + pl["N_kv"]) * D * 8 + pl["k_ctx"] * 4 + pl["n_flat"] * 4
                            + pl["n_flat"] * pl["k_ns"] * 4),
    }


# fp64 matrix-core FLOPs per launch of the selection kernels that form coarse
# scores (2*D per score): these are bound by the fp64 MFMA rate, not by HBM.
def selection_flops(p, pl):
    BH, D = p.B * p.H, p.D
    return {
        "ctx_topk_kernel": BH * 2 * D * pl["N_src"] * pl["N_ctx"],
        "sharpness_kernel": BH * 2 * D * pl["N"] * pl["N_src"],
        "flat_topk_": BH * 2 * D * pl["n_flat"] * pl["N_kv"],
    }


def kernel_times(torch, fn, reps):
    """Mean device duration (ms) of every kernel `fn` launches, from torch's
    profiler, which traces all HIP kernels of the process (the library's
    included). None when the profiler has no device activity here."""
    try:
        from torch.profiler import ProfilerActivity, profile
        fn()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
        tot, cnt = {}, {}
        for ev in prof.events():
            if str(ev.device_type).endswith("CUDA") and ev.device_time_total > 0:
                tot[ev.name] = tot.get(ev.name, 0.0) + ev.device_time_total
                cnt[ev.name] = cnt.get(ev.name, 0) + 1
        return {k: tot[k] / cnt[k] / 1e3 for k in tot} or None
    except Exception as exc:   # the profiler is context, never a reason to fail the benchmark
        log(f"kernel profiler unavailable: {exc}")
        return None


def selection_rates(torch, p, pl, fn, reps):
    """Achieved HBM GB/s of pooling and each selection kernel: algorithmic
    bytes per launch over its mean device duration (profiler), and the
    fraction of the 8 TB/s HBM peak."""
    times = kernel_times(torch, fn, reps)
    if not times:
        return None
    out = {}
    for kern, nbytes in selection_bytes(p, pl).items():
        hits = [v for k, v in times.items() if kern in k]
        if not hits:
            continue
        ms = float(np.mean(hits))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[kern] = {"ms": ms, "bytes": nbytes, "gbs": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}
        fl = selection_flops(p, pl).get(kern)
        if fl is not None:
            tf = fl / (ms * 1e-3) / 1e12
            out[kern].update({"fp64_flops": fl, "tflops": tf, "frac_of_fp64_mfma_peak": tf / PEAK_FP64_TFLOPS})
    return out


def torch_sdpa_ms(torch, Q, K, V, reps):
    """Context: PyTorch's own fused attention (flash backend only, no math
    fallback) on the same inputs, unmasked over all L tokens like the dense
    baseline. None when the installed PyTorch lacks that backend."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            o = torch.nn.functional.scaled_dot_product_attention(Q, K, V)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(max(reps, 1)):
                o = torch.nn.functional.scaled_dot_product_attention(Q, K, V)
            e1.record()
            torch.cuda.synchronize()
        del o
        return e0.elapsed_time(e1) / max(reps, 1)
    except RuntimeError:
        return None


def measured_peaks(torch, dev):
    """Achievable peaks on this device: bf16 matrix-core rate from the probe
    kernel (independent MFMA chains, no memory traffic) on random operands
    (as the attention products see) and on constant low-activity operands,
    with the shader clock each held (the matrix cores' power, so the clock,
    depends on the operand bits); HBM read bandwidth of a streaming
    16-byte-load kernel over 2 GiB, HBM bandwidth of a 2 GiB
    device-to-device copy (read + write bytes), and the LDS read rate of the
    attention kernels' two operand patterns (16-byte row reads and 8-byte
    transposed reads, 2048 workgroups of 256 threads)."""
    from block_sparse_attention_blockwise_amd import _build
    probe = ctypes.CDLL(_build.PROBE_PATH)
    probe.isa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    probe.isa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    probe.isa_probe_mfma_flops.restype = ctypes.c_double
    probe.isa_probe_wallclock_khz.restype = ctypes.c_int
    blocks, iters = 4096, 512   # about 4.5 ms per launch at 2 PFLOP/s
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall_khz = probe.isa_probe_wallclock_khz()
    mfma = {}
    for mode, name in ((1, "mfma_bf16"), (0, "mfma_bf16_low_activity")):
        rc = probe.isa_probe_mfma_bf16(blocks, iters, mode, out.data_ptr(), None, sp)
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
        for _ in range(40):   # let the clock settle under this load (about 0.2 s)
            probe.isa_probe_mfma_bf16(blocks, iters, mode, out.data_ptr(), None, sp)
        e0.record()
        for _ in range(3):
            probe.isa_probe_mfma_bf16(blocks, iters, mode, out.data_ptr(), clk.data_ptr(), sp)
        e1.record()
        torch.cuda.synchronize()
        mfma[name + "_tflops"] = 3 * probe.isa_probe_mfma_flops(blocks, iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12
        ticks = clk.view(-1, 2).double().cpu()
        ok = ticks[:, 1] > 0
        mfma[name + "_clock_ghz"] = (float((ticks[ok, 0] / ticks[ok, 1]).median()) * wall_khz * 1e-6
                                     if wall_khz > 0 and bool(ok.any()) else None)
    del clk
    n = 1 << 30   # 2^30 bf16 = 2 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    hbm_copy = 5 * 2 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    probe.isa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    rblocks = 8192
    rout = torch.empty(rblocks * 256, dtype=torch.float32, device=dev)
    rc = probe.isa_probe_read(src.data_ptr(), 2 * n, rblocks, rout.data_ptr(), sp)
    if rc != 0:
        raise RuntimeError(f"probe launch failed: {rc}")
    e0.record()
    for _ in range(5):
        probe.isa_probe_read(src.data_ptr(), 2 * n, rblocks, rout.data_ptr(), sp)
    e1.record()
    torch.cuda.synchronize()
    hbm_read = 5 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, out, rout
    probe.isa_probe_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.isa_probe_lds_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    probe.isa_probe_lds_bytes.restype = ctypes.c_double
    lblocks, liters = 2048, 4000
    lout = torch.empty(lblocks * 256, dtype=torch.float32, device=dev)
    lds = {}
    for mode, name in ((0, "lds_read_row_tbs"), (1, "lds_read_tr_tbs")):
        rc = probe.isa_probe_lds(lblocks, 16, mode, lout.data_ptr(), sp)
        if rc != 0:
            raise RuntimeError(f"probe launch failed: {rc}")
        e0.record()
        for _ in range(3):
            probe.isa_probe_lds(lblocks, liters, mode, lout.data_ptr(), sp)
        e1.record()
        torch.cuda.synchronize()
        lds[name] = 3 * probe.isa_probe_lds_bytes(lblocks, liters, mode) / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del lout
    return {**mfma, "hbm_read_gbs": hbm_read, "hbm_copy_gbs": hbm_copy, **lds}


def sweep_128k(isa, torch, dev, args):
    """The 131072-token grid (b, alpha_s, alpha_ns, alpha_f) against dense
    attention at the same length, H = 40, D = 128. Every block is full at this
    length, so the work of each point is fixed by its ratios; four generated
    heads are tiled over the 40 head slots."""
    import isa_inputs
    Ls = Lc = 65536
    H, D = 40, 128
    L = Ls + Lc
    gen = 4
    T = {n: torch.empty((1, H, L, D), dtype=torch.bfloat16, device=dev) for n in "QKV"}
    for h in range(gen):
        qkv = isa_inputs.make_head(isa_inputs.WORKLOADS["128k"]["stream"], 0, h, Ls, Lc, D)
        for n, x in zip("QKV", qkv):
            bits, _ = isa_inputs.round_to_bf16(x)
            T[n][0, h].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    for h in range(gen, H):
        for n in "QKV":
            T[n][0, h].copy_(T[n][0, h % gen])
    Q, K, V = T["Q"], T["K"], T["V"]
    O = torch.empty_like(Q)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    dense_ms = timed(lambda: isa.dense_attn(Q, K, V, out=O), 2)
    dense_flop = 4 * D * L * L * H
    rows = []
    for b in (64, 32):
        for a_s in (0.125, 0.25):
            for a_ns in (0.0625, 0.125):
                for a_f in (0.25, 0.5, 0.75):
                    p = isa.Params(1, H, Ls, Lc, D, b, a_s, a_f, a_ns)
                    pl = isa.plan(p)
                    ws = isa.workspace(p, dev)
                    ms = timed(lambda: isa.forward(Q, K, V, p, out=O, workspace=ws), 3)
                    # the two attention kernels alone, on this point's selections
                    _, sel = isa.forward(Q, K, V, p, debug=True, out=O, workspace=ws)
                    del ws
                    _, _, kcb, vcb = isa.pool_coarse(Q, K, V, p)
                    sharp_ms = timed(lambda: isa.sharp_attn(Q, K, V, sel["ctx_idx"], sel["sharp_idx"],
                                                            p, out=O), 3)
                    flat_ms = timed(lambda: isa.flat_taylor_attn(
                        Q, K, V, kcb, vcb, sel["ctx_idx"], sel["flat_idx"], sel["flat_exact_idx"],
                        p, out=O), 3)
                    del sel, kcb, vcb
                    nf, ns, nkv, kns = pl["n_flat"], pl["n_sharp"], pl["N_kv"], pl["k_ns"]
                    sharp_flop = H * 4 * D * (ns * b) * (nkv * b)
                    flat_flop = H * (4 * D * (nf * b) * (kns * b) + 4 * D * (nf * b) * (nkv - kns))
                    flop = sharp_flop + flat_flop + H * 2 * D * pl["N"] * nkv
                    rows.append({"b": b, "alpha_s": a_s, "alpha_ns": a_ns, "alpha_f": a_f, "ms": ms,
                                 "alg_tflop": flop / 1e12, "tflops": flop / (ms * 1e-3) / 1e12,
                                 "speedup_vs_dense": dense_ms / ms, "ceiling": dense_flop / flop,
                                 "sharp_ms": sharp_ms, "sharp_tflops": sharp_flop / (sharp_ms * 1e-3) / 1e12,
                                 "flat_ms": flat_ms, "flat_tflops": flat_flop / (flat_ms * 1e-3) / 1e12})
                    log(f"sweep b={b} a_s={a_s} a_ns={a_ns} a_f={a_f}: {ms:.1f} ms, "
                        f"{dense_ms / ms:.2f}x (ceiling {dense_flop / flop:.2f}x); sharp {sharp_ms:.1f} ms "
                        f"{sharp_flop / (sharp_ms * 1e-3) / 1e12:.0f} TFLOP/s, flat {flat_ms:.1f} ms "
                        f"{flat_flop / (flat_ms * 1e-3) / 1e12:.0f} TFLOP/s")
    print(json.dumps({"sweep_128k": rows, "dense_ms": dense_ms,
                      "dense_tflops": dense_flop / (dense_ms * 1e-3) / 1e12,
                      "config": {"workload": "isa_fwd_128k_tokens_h40_d128_grid"}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (the operator has no "
                                   "multi-GPU path); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import block_sparse_attention_blockwise_amd as isa

    dev = torch.device("cuda:0")
    if args.sweep:
        sweep_128k(isa, torch, dev, args)
        return
    if args.copy_calibration:
        n = 1 << 29   # 2^29 bf16 = 1 GiB
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 2 * n, "launches": max(args.steps, 1)}))
        return
    lib = isa.lib()
    w = WORKLOAD
    p = isa.Params(w["B"], w["H"], w["L_src"], w["L_ctx"], w["D"], w["b"], w["alpha_s"],
                   w["alpha_f"], w["alpha_ns"])
    pc = p.c()
    pr = ctypes.byref(pc)
    pl = isa.plan(p)
    log("generating inputs")
    T, host = make_inputs(dev)
    Q, K, V = T["Q"], T["K"], T["V"]
    if args.fig6:
        fig6(isa, torch, p, Q, K, V, args)
        return
    if args.backward:
        backward_bench(isa, torch, p, Q, K, V, args)
        return
    O = torch.empty_like(Q)
    BH = p.B * p.H
    e = lambda *s, dt: torch.empty(s, dtype=dt, device=dev)
    qc = e(BH, pl["N"], p.D, dt=torch.float64)
    kc = e(BH, pl["N"], p.D, dt=torch.float64)
    kcb = e(BH, pl["N"], p.D, dt=torch.bfloat16)
    vcb = e(BH, pl["N"], p.D, dt=torch.bfloat16)
    ctx = e(BH, pl["k_ctx"], dt=torch.int32)
    score = e(BH, pl["N_ctx"], dt=torch.float64)
    sharp = e(BH, pl["N"], dt=torch.float64)
    si = e(BH, pl["n_sharp"], dt=torch.int32)
    fi = e(BH, pl["n_flat"], dt=torch.int32)
    ei = e(BH, pl["n_flat"], pl["k_ns"], dt=torch.int32)
    ws_s = e(pl["scores_bytes"], dt=torch.uint8)
    ws_f = e(pl["workspace_bytes"], dt=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def chk(name, rc):
        if rc != 0:
            raise RuntimeError(f"{name}: {isa.strerror(rc)}")

    names = ["pool", "ctx_topk", "sharpness_split", "sharp_attn", "flat_taylor_attn"]

    def step(ev=None):
        if ev: ev[0].record(stream)
        chk("pool", lib.isa_pool_coarse(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), qc.data_ptr(),
                                        kc.data_ptr(), kcb.data_ptr(), vcb.data_ptr(), sp))
        if ev: ev[1].record(stream)
        chk("ctx", lib.isa_ctx_topk(pr, qc.data_ptr(), kc.data_ptr(), ctx.data_ptr(), score.data_ptr(), sp))
        if ev: ev[2].record(stream)
        chk("split", lib.isa_sharpness_split(pr, qc.data_ptr(), kc.data_ptr(), ctx.data_ptr(),
                                             sharp.data_ptr(), si.data_ptr(), fi.data_ptr(),
                                             ei.data_ptr(), ws_s.data_ptr(), ws_s.numel(), sp))
        if ev: ev[3].record(stream)
        chk("sharp", lib.isa_sharp_attn(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), ctx.data_ptr(),
                                        si.data_ptr(), O.data_ptr(), sp))
        if ev: ev[4].record(stream)
        chk("flat", lib.isa_flat_taylor_attn(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), kcb.data_ptr(),
                                             vcb.data_ptr(), ctx.data_ptr(), fi.data_ptr(), ei.data_ptr(),
                                             O.data_ptr(), sp))
        if ev: ev[5].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    if args.only == "sharp":
        for _ in range(args.steps):
            chk("sharp", lib.isa_sharp_attn(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), ctx.data_ptr(),
                                            si.data_ptr(), O.data_ptr(), sp))
        torch.cuda.synchronize()
        print(json.dumps({"only": "sharp", "launches": args.steps}))
        return
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {n: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]))
           for i, n in enumerate(names)}
    step_ms = float(np.mean([evs[k][0].elapsed_time(evs[k][5]) for k in range(args.steps)]))
    p10, p90 = (float(x) for x in np.percentile(
        [evs[k][0].elapsed_time(evs[k][5]) for k in range(args.steps)], [10, 90]))

    # isa_forward (same kernels, one call)
    fwd_ms = None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        chk("fwd", lib.isa_forward(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                   ws_f.data_ptr(), ws_f.numel(), None, sp))
    e0.record(stream)
    for _ in range(args.steps):
        chk("fwd", lib.isa_forward(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                   ws_f.data_ptr(), ws_f.numel(), None, sp))
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / args.steps
    # the decomposed step (five entry points) must produce what isa_forward does
    O_fwd = O.clone()
    step()
    torch.cuda.synchronize()
    same = bool(torch.equal(O_fwd.view(torch.int16), O.view(torch.int16)))

    # backward of the same forward (dO ~ N(0, 1)): isa_forward saves its state in
    # ws_f, isa_backward reuses it
    g = torch.Generator(device=dev).manual_seed(5)
    dO = torch.randn(Q.shape, device=dev, generator=g).to(torch.bfloat16)
    gQ, gK, gV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)

    def fwd_bwd():
        chk("fwd", lib.isa_forward(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                   ws_f.data_ptr(), ws_f.numel(), None, sp))
        e0.record(stream)
        chk("bwd", lib.isa_backward(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                                    dO.data_ptr(), gQ.data_ptr(), gK.data_ptr(), gV.data_ptr(),
                                    ws_f.data_ptr(), ws_f.numel(), sp))
        e1.record(stream)
    fwd_bwd()
    bwd_ms = 0.0
    nb = max(args.steps // 5, 2)
    for _ in range(nb):
        fwd_bwd()
        torch.cuda.synchronize()
        bwd_ms += e0.elapsed_time(e1) / nb
    del dO, gQ, gK, gV

    # decoupled RoPE fused with pooling (same workload, base 10000): reads Q, K, V
    # once, writes the rotated Q and K and the block means
    pr_rope = isa.Params(p.B, p.H, p.L_src, p.L_ctx, p.D, p.b, p.alpha_s, p.alpha_f, p.alpha_ns,
                         rope_base=10000.0)
    prc = pr_rope.c()
    Qr, Kr = torch.empty_like(Q), torch.empty_like(K)
    ws_r = e(max(isa.plan(pr_rope)["rope_bytes"], 1), dt=torch.uint8)

    def rope_pool():
        chk("rope", lib.isa_rope_pool_coarse(ctypes.byref(prc), Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                             Qr.data_ptr(), Kr.data_ptr(), qc.data_ptr(), kc.data_ptr(),
                                             kcb.data_ptr(), vcb.data_ptr(), ws_r.data_ptr(),
                                             ws_r.numel(), sp))
    rope_pool()
    e0.record(stream)
    for _ in range(args.steps):
        rope_pool()
    e1.record(stream)
    torch.cuda.synchronize()
    rope_ms = e0.elapsed_time(e1) / args.steps
    del Qr, Kr, ws_r

    # residual gamma * O_coarse (gamma = 0.5, same workload): the step on its
    # own (adds into O in place) and the whole forward with it
    pg = isa.Params(p.B, p.H, p.L_src, p.L_ctx, p.D, p.b, p.alpha_s, p.alpha_f, p.alpha_ns, gamma=0.5)
    pgc = pg.c()
    ws_g = e(isa.plan(pg)["workspace_bytes"], dt=torch.uint8)
    ws_res = e(isa.plan(pg)["scores_bytes"], dt=torch.uint8)   # the residual's coarse rows

    def residual():
        chk("residual", lib.isa_coarse_residual(ctypes.byref(pgc), qc.data_ptr(), kc.data_ptr(), vcb.data_ptr(),
                                                ctx.data_ptr() if ctx.numel() else None, O.data_ptr(),
                                                ws_res.data_ptr(), ws_res.numel(), sp))

    def forward_residual():
        chk("fwd_residual", lib.isa_forward(ctypes.byref(pgc), Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                            O.data_ptr(), ws_g.data_ptr(), ws_g.numel(), None, sp))
    timings = {}
    for name, fn in (("residual", residual), ("forward_residual", forward_residual)):
        fn()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        timings[name] = e0.elapsed_time(e1) / args.steps
    del ws_g, ws_res

    # pooling and the selection kernels one by one (per-kernel durations)
    def selection_step():
        chk("pool", lib.isa_pool_coarse(pr, Q.data_ptr(), K.data_ptr(), V.data_ptr(), qc.data_ptr(),
                                        kc.data_ptr(), kcb.data_ptr(), vcb.data_ptr(), sp))
        chk("ctx", lib.isa_ctx_topk(pr, qc.data_ptr(), kc.data_ptr(), ctx.data_ptr(), score.data_ptr(), sp))
        chk("split", lib.isa_sharpness_split(pr, qc.data_ptr(), kc.data_ptr(), ctx.data_ptr(),
                                             sharp.data_ptr(), si.data_ptr(), fi.data_ptr(),
                                             ei.data_ptr(), ws_s.data_ptr(), ws_s.numel(), sp))
    sel_rates = selection_rates(torch, p, pl, selection_step, 5)

    flops = algorithmic_flops(p, pl, ctx.view(p.B, p.H, -1).cpu().numpy(),
                              si.view(p.B, p.H, -1).cpu().numpy(), fi.view(p.B, p.H, -1).cpu().numpy(),
                              ei.view(p.B, p.H, pl["n_flat"], pl["k_ns"]).cpu().numpy())
    alg_total = flops["sharp"] + flops["flat_exact"] + flops["taylor"] + flops["coarse"]

    dense_ms = None
    if not args.no_dense:
        log("dense baseline")
        isa.dense_attn(Q, K, V, out=O)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.dense_reps):
            chk("dense", lib.isa_dense_attn(p.B, p.H, p.L_src + p.L_ctx, p.D, Q.data_ptr(), K.data_ptr(),
                                            V.data_ptr(), O.data_ptr(), sp))
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_reps
    sdpa_ms = None if args.no_dense else torch_sdpa_ms(torch, Q, K, V, args.dense_reps)

    sharp_tflops = flops["sharp"] / (per["sharp_attn"] * 1e-3) / 1e12
    rec = traffic_record()
    peaks = measured_peaks(torch, dev)
    roofline = {"bound": "mfma", "kernel": "isa_sharp_attn (attn_kernel<128,sharp>)",
                "achieved": sharp_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": sharp_tflops / PEAK_BF16_TFLOPS, "traffic": rec,
                "algorithmic_flops_per_launch": flops["sharp"],
                "avg_launch_ms": per["sharp_attn"],
                "measured_peak": peaks["mfma_bf16_tflops"],
                "frac_of_measured_peak": sharp_tflops / peaks["mfma_bf16_tflops"]}
    pool_bytes = 3 * BH * (p.L_src + p.L_ctx) * p.D * 2 + BH * pl["N"] * p.D * (8 + 8 + 2 + 2)
    out = {
        "metric": METRIC, "value": step_ms, "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded clustered generator)",
        "config": {"workload": "isa_fwd_64k_tokens_h40_d128", "B": p.B, "H": p.H, "L_src": p.L_src,
                   "L_ctx": p.L_ctx, "D": p.D, "b": p.b, "alpha_s": p.alpha_s,
                   "alpha_f": p.alpha_f, "alpha_ns": p.alpha_ns},
        "latency_p10_p90_ms": [p10, p90],
        "wall_ms_per_step": wall_ms,
        "isa_forward_ms": fwd_ms,
        "forward_matches_steps": same,
        "per_kernel_ms": per,
        "tflops_dense_equivalent": flops["dense"] / (step_ms * 1e-3) / 1e12,
        "tflops_algorithmic": alg_total / (step_ms * 1e-3) / 1e12,
        "mfma_util": {"sharp_attn": sharp_tflops / PEAK_BF16_TFLOPS,
                      "flat_taylor_attn": (flops["flat_exact"] + flops["taylor"]) /
                      (per["flat_taylor_attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "pool_hbm_frac": pool_bytes / (per["pool"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "pool_hbm_frac_of_measured_read": pool_bytes / (per["pool"] * 1e-3) / 1e9 / peaks["hbm_read_gbs"],
        "measured_peaks": peaks,
        "selection_hbm": sel_rates,
        "isa_backward_ms": bwd_ms,
        "rope_pool_ms": rope_ms,
        "coarse_residual_ms": timings["residual"],
        "isa_forward_residual_ms": timings["forward_residual"],
        "rope_pool_hbm_frac": (pool_bytes + 2 * BH * (p.L_src + p.L_ctx) * p.D * 2) /
                              (rope_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_tflop": {k: v / 1e12 for k, v in flops.items()},
        "dense_ms": dense_ms,
        "dense_tflops": (flops["dense"] / (dense_ms * 1e-3) / 1e12) if dense_ms else None,
        "speedup_vs_dense": (dense_ms / step_ms) if dense_ms else None,
        "torch_sdpa_flash_ms": sdpa_ms,
        "speedup_vs_torch_sdpa": (sdpa_ms / step_ms) if sdpa_ms else None,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(host, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
