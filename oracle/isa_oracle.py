"""Blockwise fp64 CPU oracle for the In-context Sparse Attention (ISA) forward pass.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module. The HIP library never
calls it, and it shares no code with the HIP path.

What it computes, per (batch, head), written from these pages:

* [RB] paper.rainbus.top structured summary of arXiv 2605.04569
  ("LIVEditor-14B ... In-Context Sparse Attention"), sections "Prerequisites"
  (block-sparse and pooling attention; 0th-order Taylor attention), "Core
  method" and "Method steps" steps (1)-(6).
* [TW] techwalker.com news article on the same paper, section 4 (the ISA
  workflow) and section 5 (block-wise 0th-order Taylor sparse attention).
* [HF] the LIVEditor model card, section "Method".

ISA is an approximation, so the oracle is the algorithm itself, step by
step, in float64, on the exact input values given to the GPU (bf16 values
widened to fp64). Outputs are computed with a max-shifted two-pass softmax.

Readings where the pages are silent or contradict each other (each is
listed with its reason in the repository's design notes):

R1  alpha_f is the fraction of query blocks sent to the flat (Taylor) path
    ([RB] "Method steps" step (3)); alpha_s=1, alpha_f=0 is then dense
    attention.
R2  counts round toward more exact work: k_ctx = ceil(alpha_s*N_ctx),
    n_flat = floor(alpha_f*N), k_ns = min(N_kv, ceil(alpha_ns*N_kv)).
R3  blocks are cut per segment (source, then context), each tail block holds
    the remaining n_j < b tokens, and means are over the n_j valid tokens.
R4  sharpness of query block i is the population variance of the softmax of
    its coarse scores over the source key-block columns.
R5  every query block (source and context) gets a sharpness and a path.
R6  the context score is the raw scaled coarse score summed over the source
    query rows.
R7  the sharp and the flat path both see only the kept KV blocks J (all
    source blocks plus the selected context blocks); pruned context blocks
    contribute nothing, and the "total block count" for alpha_ns is |J|.
R8  the exact set E_i of a flat block is the top k_ns of its coarse row over
    J; the Taylor weight of block j is n_j (the step (5) factor L_K), applied
    to numerator and denominator.
R9  the low-frequency residual of step (6) is gamma * O_coarse, with
    O_coarse_i = softmax over the kept blocks J of the coarse row S[i, J]
    applied to Vc[J] (the pooled attention of step (1) at block resolution,
    unweighted), broadcast to every token of block i. The pages never give
    gamma; the default is 0 (residual off).
R10 ties: the lower index wins in every top-k; in the split a lower index
    counts as sharper.
R11 decoupled RoPE (the step before (1), [RB] "Novelty"; [TW] section 6):
    standard rotary embedding of Q and K on interleaved pairs (2i, 2i+1)
    with angle pos * base^(-2i/D), where source tokens take positions
    0..L_src-1 and context tokens restart at 0. The pages give no base and
    no precision; the rotated tensors are the attention inputs, so they are
    stored as bf16: cos/sin are computed in fp64 and rounded to fp32, the
    rotation is done in fp32 with each product and sum rounded, and the
    result is rounded to bf16 (the arithmetic of the kernel, so both sides
    produce the same bf16 values).
R12 backward (trainable ISA, [RB] "Core method" and Novelty (c): the
    operator is trained end to end): the selections are piecewise constant
    in Q, K, V, so gradients flow only through the attention terms with the
    selections held fixed; the exact terms give the usual softmax-attention
    gradients, the Taylor terms reach K and V through the block means
    (each token of block j receives 1/n_j of the gradient of Kc_j, Vc_j),
    and, when gamma != 0, the residual reaches Q, K, V through Qc, Kc, Vc.
    The bf16 roundings of the forward (rotated Q/K, the Taylor operands) are
    taken as the identity.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_EPS_ROUND = 1e-9


# ---------------------------------------------------------------- counts (R2)
def _ceil(x: float) -> int:
    return int(math.ceil(x - _EPS_ROUND))


def _floor(x: float) -> int:
    return int(math.floor(x + _EPS_ROUND))


@dataclass(frozen=True)
class Plan:
    L_src: int
    L_ctx: int
    b: int
    N_src: int
    N_ctx: int
    N: int
    k_ctx: int
    N_kv: int
    n_flat: int
    n_sharp: int
    k_ns: int
    starts: tuple = field(repr=False)
    counts: tuple = field(repr=False)


def make_plan(L_src: int, L_ctx: int, b: int, alpha_s: float, alpha_f: float,
              alpha_ns: float) -> Plan:
    """Block partition and selection counts.

    [RB] "Method steps" step (1) cuts Q/K/V into b-token blocks with padding;
    step (2) keeps alpha_s * ceil(L_ctx/b) context blocks; step (3) routes a
    fraction alpha_f of query blocks to the flat path; step (5) computes
    alpha_ns * (block count) blocks exactly per flat query block.
    """
    if L_src < 1 or L_ctx < 0 or b < 1:
        raise ValueError("need L_src >= 1, L_ctx >= 0, b >= 1")
    for a in (alpha_s, alpha_f, alpha_ns):
        if not (0.0 <= a <= 1.0):
            raise ValueError("ratios must lie in [0, 1]")
    N_src = -(-L_src // b)
    N_ctx = -(-L_ctx // b)
    N = N_src + N_ctx
    k_ctx = min(N_ctx, _ceil(alpha_s * N_ctx))
    N_kv = N_src + k_ctx
    n_flat = min(N, _floor(alpha_f * N))
    k_ns = min(N_kv, _ceil(alpha_ns * N_kv))
    starts, counts = [], []
    # R3: source blocks first, then context blocks; no block straddles the
    # source/context boundary.
    for j in range(N_src):
        starts.append(j * b)
        counts.append(min(b, L_src - j * b))
    for j in range(N_ctx):
        starts.append(L_src + j * b)
        counts.append(min(b, L_ctx - j * b))
    return Plan(L_src, L_ctx, b, N_src, N_ctx, N, k_ctx, N_kv, n_flat, N - n_flat,
                k_ns, tuple(starts), tuple(counts))


# ------------------------------------------------------ decoupled RoPE (R11)
def rope_positions(L_src: int, L_ctx: int) -> np.ndarray:
    """Source tokens 0..L_src-1, context tokens restarting at 0."""
    return np.concatenate([np.arange(L_src), np.arange(L_ctx)]).astype(np.float64)


def rope_tables(pos: np.ndarray, D: int, base: float):
    """cos/sin of pos * base^(-2i/D) for i < D/2: fp64, then rounded to fp32."""
    inv = base ** (-(2.0 * np.arange(D // 2)) / D)
    ang = pos[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32)


def rope(X: np.ndarray, L_src: int, L_ctx: int, base: float) -> np.ndarray:
    """Rotates X [L, D] pairwise (R11); returns the bf16 result as float64."""
    X = np.asarray(X, dtype=np.float32)
    c, s = rope_tables(rope_positions(L_src, L_ctx), X.shape[1], base)
    x, y = X[:, 0::2], X[:, 1::2]
    xr = (x * c).astype(np.float32) - (y * s).astype(np.float32)
    yr = (x * s).astype(np.float32) + (y * c).astype(np.float32)
    out = np.empty_like(X)
    out[:, 0::2] = xr
    out[:, 1::2] = yr
    return _bf16_rne(out).astype(np.float64)


# ------------------------------------------------------------ selection steps
def pool(X: np.ndarray, plan: Plan) -> np.ndarray:
    """Mean of each block's valid tokens ([RB] step (1); R3). X is [L, D]."""
    X = np.asarray(X, dtype=np.float64)
    out = np.empty((plan.N, X.shape[1]), dtype=np.float64)
    for j, (s, n) in enumerate(zip(plan.starts, plan.counts)):
        out[j] = X[s:s + n].mean(axis=0)
    return out


def coarse_scores(Qc: np.ndarray, Kc: np.ndarray) -> np.ndarray:
    """S = Qc Kc^T / sqrt(D) at block resolution ([RB] step (1))."""
    D = Qc.shape[1]
    return (Qc @ Kc.T) / math.sqrt(D)


def context_scores(S: np.ndarray, plan: Plan) -> np.ndarray:
    """Importance of each context block: its coarse-score column summed over
    the source query rows ([RB] step (2); R6)."""
    return S[:plan.N_src, plan.N_src:].sum(axis=0)


def top_k(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, lower index first on ties (R10),
    returned sorted ascending."""
    scores = np.asarray(scores, dtype=np.float64)
    order = np.lexsort((np.arange(scores.size), -scores))
    return np.sort(order[:k]).astype(np.int64)


def sharpness(S: np.ndarray, plan: Plan) -> np.ndarray:
    """M_i = Var(softmax(S[i, source columns])) ([RB] "Core method" and step (3);
    R4, R5). Population variance over the N_src probabilities."""
    x = S[:, :plan.N_src]
    x = x - x.max(axis=1, keepdims=True)
    e = np.exp(x)
    p = e / e.sum(axis=1, keepdims=True)
    return ((p - 1.0 / plan.N_src) ** 2).mean(axis=1)


def split(M: np.ndarray, plan: Plan):
    """Rank blocks by descending sharpness (ties: lower index sharper, R10);
    the first n_sharp are sharp, the rest flat ([RB] step (3); R1).
    Both lists are returned sorted ascending."""
    order = np.lexsort((np.arange(M.size), -M))
    return np.sort(order[:plan.n_sharp]).astype(np.int64), np.sort(order[plan.n_sharp:]).astype(np.int64)


def kept_blocks(ctx_idx: np.ndarray, plan: Plan) -> np.ndarray:
    """J: every source block plus the selected context blocks ([RB] step (2):
    source KV concatenated with the gathered context KV), ascending global ids."""
    return np.concatenate([np.arange(plan.N_src), plan.N_src + np.asarray(ctx_idx, dtype=np.int64)])


def exact_sets(S: np.ndarray, J: np.ndarray, flat_idx: np.ndarray, plan: Plan) -> np.ndarray:
    """E_i for every flat block i: the k_ns blocks of J with the largest coarse
    score S[i, j] ([RB] step (5); R8, R10). Rows aligned with flat_idx,
    each sorted ascending (global block ids)."""
    out = np.empty((len(flat_idx), plan.k_ns), dtype=np.int64)
    for r, i in enumerate(flat_idx):
        sel = top_k(S[i, J], plan.k_ns)
        out[r] = np.sort(J[sel])
    return out


def _topk_gap(scores: np.ndarray, k: int) -> float:
    """Score of the k-th kept element minus the best dropped one (inf if
    nothing is dropped or nothing kept). This is the margin by which a top-k
    selection is decided: below the parity tie band two valid selections may
    differ."""
    if k <= 0 or k >= scores.size:
        return math.inf
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    return float(s[k - 1] - s[k])


def _split_gap(M: np.ndarray, plan: Plan) -> float:
    """Margin of the sharp/flat split ([RB] step (3)): the top-n_sharp gap of
    the normalised sharpness N_src^2 * M_i (0 for a uniform softmax row,
    N_src - 1 for a one-hot row), inf when every block is on one path."""
    if plan.n_flat in (0, plan.N):
        return math.inf
    return _topk_gap(np.asarray(M, dtype=np.float64) * plan.N_src ** 2, plan.n_sharp)


def _exact_gaps(S: np.ndarray, J: np.ndarray, flat_idx: np.ndarray, plan: Plan) -> np.ndarray:
    """Margin of each flat block's exact-set choice ([RB] step (5)): the
    top-k_ns gap of its coarse row over the kept blocks J, aligned with
    flat_idx."""
    return np.array([_topk_gap(S[i, J], plan.k_ns) for i in flat_idx], dtype=np.float64)


# --------------------------------------------------------------- attention
def _token_range(plan: Plan, j: int) -> np.ndarray:
    s = plan.starts[j]
    return np.arange(s, s + plan.counts[j])


def _sharp_block_out(Qi, K, V, key_tok, D):
    """Exact softmax attention of Qi over the listed key tokens
    ([RB] step (4)), two-pass max-shifted. key_tok None: K and V already hold
    exactly the listed key rows."""
    Kx = K if key_tok is None else K[key_tok]
    Vx = V if key_tok is None else V[key_tok]
    logits = (Qi @ Kx.T) / math.sqrt(D)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    return (w @ Vx) / w.sum(axis=1, keepdims=True)


def _flat_block_out(Qi, K, V, Kc, Vc, exact_tok, taylor_blocks, n_taylor, D):
    """[RB] step (5) and the 0th-order Taylor paragraph of "Prerequisites";
    [TW] section 5: exact terms for the tokens of E_i, and for every other
    kept block j the term n_j * exp(q . Kc_j / sqrt(D)) added to the
    denominator and that weight times Vc_j to the numerator (R8)."""
    scale = 1.0 / math.sqrt(D)
    le = (Qi @ K[exact_tok].T) * scale
    lt = (Qi @ Kc[taylor_blocks].T) * scale
    m = np.full((Qi.shape[0], 1), -np.inf)
    if le.size:
        m = np.maximum(m, le.max(axis=1, keepdims=True))
    if lt.size:
        m = np.maximum(m, lt.max(axis=1, keepdims=True))
    we = np.exp(le - m)
    wt = np.exp(lt - m) * n_taylor[None, :]
    num = we @ V[exact_tok] + wt @ Vc[taylor_blocks]
    den = we.sum(axis=1, keepdims=True) + wt.sum(axis=1, keepdims=True)
    return num / den


@dataclass
class HeadResult:
    O: np.ndarray               # [L, D] float64 (rows not requested are NaN)
    ctx_idx: np.ndarray         # [k_ctx] context-local ids, ascending
    sharp_idx: np.ndarray       # [n_sharp] ascending
    flat_idx: np.ndarray        # [n_flat] ascending
    flat_exact_idx: np.ndarray  # [n_flat, k_ns] global ids, rows ascending
    ctx_score: np.ndarray       # [N_ctx]
    sharpness: np.ndarray       # [N]
    S: np.ndarray               # [N, N] coarse scores
    Qc: np.ndarray
    Kc: np.ndarray
    Vc: np.ndarray
    ctx_gap: float
    split_gap: float            # on normalised sharpness N_src^2 * M
    exact_gaps: np.ndarray      # [n_flat]


def coarse_output(S: np.ndarray, Vc: np.ndarray, J: np.ndarray) -> np.ndarray:
    """O_coarse [N, D]: for query block i, softmax(S[i, J]) applied to Vc[J]
    ([RB] "Method steps" step (6), reading R9)."""
    x = S[:, J]
    x = x - x.max(axis=1, keepdims=True)
    w = np.exp(x)
    return (w @ Vc[J]) / w.sum(axis=1, keepdims=True)


def isa_head(Q, K, V, plan: Plan, selections: dict | None = None, rows=None,
             compute_output: bool = True, gamma: float = 0.0) -> HeadResult:
    """ISA forward for one (batch, head). Q, K, V: [L, D] arrays.

    `selections` may inject ctx_idx / sharp_idx / flat_idx / flat_exact_idx
    (used when a selection legitimately differs inside a score tie band);
    the remaining steps then use the injected lists. `rows` restricts the
    output to the given token indices (others are NaN).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, D = Q.shape
    assert L == plan.L_src + plan.L_ctx
    sel = selections or {}

    Qc, Kc, Vc = pool(Q, plan), pool(K, plan), pool(V, plan)
    S = coarse_scores(Qc, Kc)
    r = context_scores(S, plan)
    ctx_idx = np.asarray(sel["ctx_idx"], dtype=np.int64) if "ctx_idx" in sel else top_k(r, plan.k_ctx)
    J = kept_blocks(ctx_idx, plan)
    M = sharpness(S, plan)
    if "sharp_idx" in sel:
        sharp_idx = np.asarray(sel["sharp_idx"], dtype=np.int64)
        flat_idx = np.asarray(sel["flat_idx"], dtype=np.int64)
    else:
        sharp_idx, flat_idx = split(M, plan)
    E = (np.asarray(sel["flat_exact_idx"], dtype=np.int64) if "flat_exact_idx" in sel
         else exact_sets(S, J, flat_idx, plan))

    split_gap = _split_gap(M, plan)
    exact_gaps = _exact_gaps(S, J, flat_idx, plan)

    O = np.full((L, D), np.nan)
    if compute_output:
        want = None if rows is None else np.zeros(L, dtype=bool)
        if want is not None:
            want[np.asarray(rows, dtype=np.int64)] = True
        counts = np.asarray(plan.counts, dtype=np.float64)
        J_tok = np.concatenate([_token_range(plan, j) for j in J])
        KJ, VJ = K[J_tok], V[J_tok]          # the key rows of J, gathered once
        for i in sharp_idx:
            tok = _token_range(plan, i)
            if want is not None:
                tok = tok[want[tok]]
            if tok.size:
                O[tok] = _sharp_block_out(Q[tok], KJ, VJ, None, D)
        for rix, i in enumerate(flat_idx):
            tok = _token_range(plan, i)
            if want is not None:
                tok = tok[want[tok]]
            if not tok.size:
                continue
            Ei = E[rix]
            Ti = np.setdiff1d(J, Ei)
            exact_tok = (np.concatenate([_token_range(plan, j) for j in Ei])
                         if Ei.size else np.zeros(0, dtype=np.int64))
            O[tok] = _flat_block_out(Q[tok], K, V, Kc, Vc, exact_tok, Ti, counts[Ti], D)
        if gamma != 0.0:
            Oc = coarse_output(S, Vc, J)
            for i in range(plan.N):
                tok = _token_range(plan, i)
                O[tok] += gamma * Oc[i][None, :]

    return HeadResult(O, ctx_idx, sharp_idx, flat_idx, E, r, M, S, Qc, Kc, Vc,
                      _topk_gap(r, plan.k_ctx), split_gap, exact_gaps)


# ---------------------------------------------------------------- backward
def _attn_rows_backward(Qi, dOi, Kx, Vx, bias, scale):
    """Gradients of o = softmax(scale * Qi Kx^T + bias) Vx for one set of
    query rows against its key rows (bias: additive logit per key row).
    Returns (dQi, dKx, dVx) with the softmax Jacobian written out:
    dS = P * (dO Vx^T - rowsum(dO * o))."""
    logits = (Qi @ Kx.T) * scale + bias[None, :]
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    P = w / w.sum(axis=1, keepdims=True)
    O = P @ Vx
    dS = P * (dOi @ Vx.T - (dOi * O).sum(axis=1, keepdims=True))
    return (dS @ Kx) * scale, (dS.T @ Qi) * scale, P.T @ dOi


def isa_head_backward(Q, K, V, dO, plan: Plan, selections: dict | None = None,
                      gamma: float = 0.0):
    """Gradients (dQ, dK, dV) [L, D] fp64 of sum(dO * O) for one (batch,
    head), O the ISA output of isa_head with the same selections (R12)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    L, D = Q.shape
    scale = 1.0 / math.sqrt(D)
    f = isa_head(Q, K, V, plan, selections=selections, compute_output=False)
    J = kept_blocks(f.ctx_idx, plan)
    counts = np.asarray(plan.counts, dtype=np.float64)
    dQ, dK, dV = np.zeros((L, D)), np.zeros((L, D)), np.zeros((L, D))
    dQc, dKc, dVc = np.zeros((plan.N, D)), np.zeros((plan.N, D)), np.zeros((plan.N, D))
    J_tok = np.concatenate([_token_range(plan, j) for j in J])
    for i in f.sharp_idx:                       # step (4): exact over the tokens of J
        tok = _token_range(plan, i)
        gq, gk, gv = _attn_rows_backward(Q[tok], dO[tok], K[J_tok], V[J_tok],
                                         np.zeros(J_tok.size), scale)
        dQ[tok] += gq
        dK[J_tok] += gk
        dV[J_tok] += gv
    for r, i in enumerate(f.flat_idx):          # step (5): exact over E_i, Taylor over J \ E_i
        tok = _token_range(plan, i)
        Ei = f.flat_exact_idx[r]
        Ti = np.setdiff1d(J, Ei)
        ex = (np.concatenate([_token_range(plan, j) for j in Ei]) if Ei.size
              else np.zeros(0, dtype=np.int64))
        Kx = np.vstack([K[ex], f.Kc[Ti]])
        Vx = np.vstack([V[ex], f.Vc[Ti]])
        bias = np.concatenate([np.zeros(ex.size), np.log(counts[Ti])])
        gq, gk, gv = _attn_rows_backward(Q[tok], dO[tok], Kx, Vx, bias, scale)
        dQ[tok] += gq
        dK[ex] += gk[:ex.size]
        dV[ex] += gv[:ex.size]
        dKc[Ti] += gk[ex.size:]
        dVc[Ti] += gv[ex.size:]
    if gamma != 0.0:                            # step (6) residual on the pooled rows
        dOc = np.stack([dO[_token_range(plan, i)].sum(axis=0) for i in range(plan.N)]) * gamma
        gq, gk, gv = _attn_rows_backward(f.Qc, dOc, f.Kc[J], f.Vc[J], np.zeros(J.size), scale)
        dQc += gq
        dKc[J] += gk
        dVc[J] += gv
    for j in range(plan.N):                     # through the block means of step (1)
        tok = _token_range(plan, j)
        dQ[tok] += dQc[j] / counts[j]
        dK[tok] += dKc[j] / counts[j]
        dV[tok] += dVc[j] / counts[j]
    return dQ, dK, dV


def isa_head_dq_rows(Q, K, V, dO, plan: Plan, rows, selections: dict | None = None):
    """dQ of the listed token rows only (gamma = 0), [len(rows), D] fp64: each
    row's own softmax over its key set gives its dQ (R12), so large shapes can
    be sampled row by row."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    D = Q.shape[1]
    scale = 1.0 / math.sqrt(D)
    f = isa_head(Q, K, V, plan, selections=selections, compute_output=False)
    J = kept_blocks(f.ctx_idx, plan)
    counts = np.asarray(plan.counts, dtype=np.float64)
    J_tok = np.concatenate([_token_range(plan, j) for j in J])
    block_of = np.concatenate([np.full(n, j) for j, n in enumerate(plan.counts)])
    flat_row = {int(i): r for r, i in enumerate(f.flat_idx)}
    out = np.empty((len(rows), D))
    for k, t in enumerate(np.asarray(rows, dtype=np.int64)):
        i = int(block_of[t])
        if i in flat_row:
            Ei = f.flat_exact_idx[flat_row[i]]
            Ti = np.setdiff1d(J, Ei)
            ex = (np.concatenate([_token_range(plan, j) for j in Ei]) if Ei.size
                  else np.zeros(0, dtype=np.int64))
            Kx = np.vstack([K[ex], f.Kc[Ti]])
            Vx = np.vstack([V[ex], f.Vc[Ti]])
            bias = np.concatenate([np.zeros(ex.size), np.log(counts[Ti])])
        else:
            Kx, Vx, bias = K[J_tok], V[J_tok], np.zeros(J_tok.size)
        gq, _, _ = _attn_rows_backward(Q[t:t + 1], dO[t:t + 1], Kx, Vx, bias, scale)
        out[k] = gq[0]
    return out


def rope_backward(dXr: np.ndarray, L_src: int, L_ctx: int, base: float) -> np.ndarray:
    """Gradient through the rotation of R11 (the transpose of each 2x2
    rotation, with the same fp32 cos/sin values), fp64, rounding taken as
    the identity (R12)."""
    dXr = np.asarray(dXr, dtype=np.float64)
    c, s = rope_tables(rope_positions(L_src, L_ctx), dXr.shape[1], base)
    c, s = c.astype(np.float64), s.astype(np.float64)
    gx, gy = dXr[:, 0::2], dXr[:, 1::2]
    out = np.empty_like(dXr)
    out[:, 0::2] = gx * c + gy * s
    out[:, 1::2] = gy * c - gx * s
    return out


def isa_forward(Q, K, V, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns, heads=None, gamma=0.0):
    """ISA over [B, H, L, D] inputs; returns (O [B,H,L,D] float64, results
    dict keyed by (b_idx, h)). `heads` restricts the work to listed heads."""
    plan = make_plan(L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns)
    Bn, Hn, L, D = np.shape(Q)
    O = np.full((Bn, Hn, L, D), np.nan)
    res = {}
    for (bi, h) in (heads if heads is not None else [(x, y) for x in range(Bn) for y in range(Hn)]):
        hr = isa_head(Q[bi, h], K[bi, h], V[bi, h], plan, gamma=gamma)
        O[bi, h] = hr.O
        res[(bi, h)] = hr
    return O, res


def dense_attention(Q, K, V, rows=None) -> np.ndarray:
    """softmax(Q K^T / sqrt(D)) V over every token (no mask), fp64; the
    dense baseline the pages measure against ([RB] "Prerequisites",
    SDPA and FlashAttention paragraph)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, D = Q.shape
    idx = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.full((L, D), np.nan)
    for s in range(0, idx.size, 256):
        t = idx[s:s + 256]
        out[t] = _sharp_block_out(Q[t], K, V, np.arange(L), D)
    return out
