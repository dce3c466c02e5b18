"""Token-level brute-force ISA, written independently of the blockwise oracle.

TEST INFRASTRUCTURE ONLY (same rule as the blockwise oracle: imported by the
tests alone). It shares no helper with isa_oracle.py and is meant for tiny
inputs: explicit per-token loops, selections by rank counting instead of
sorting, and the context top-k by enumerating every subset.

Sources: the rainbus.top summary of arXiv 2605.04569, section "Method
steps" steps (1)-(5), and its "Prerequisites" paragraph on the 0th-order
Taylor approximation; same readings R1-R10 as the blockwise oracle.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _blocks(L_src, L_ctx, b):
    """List of (first token, token count) per block, source segment then
    context segment, walked token by token."""
    out = []
    for seg0, seg_len in ((0, L_src), (L_src, L_ctx)):
        t = 0
        while t < seg_len:
            n = 0
            while n < b and t + n < seg_len:
                n += 1
            out.append((seg0 + t, n))
            t += n
    return out


def _mean_loop(X, s, n):
    D = X.shape[1]
    acc = [0.0] * D
    for t in range(s, s + n):
        for d in range(D):
            acc[d] += float(X[t, d])
    return [a / n for a in acc]


def _dot(a, b):
    return math.fsum(float(x) * float(y) for x, y in zip(a, b))


def _rank_select(values, k):
    """Element i is selected iff fewer than k elements beat it, where j beats
    i when values[j] > values[i], or values[j] == values[i] and j < i."""
    n = len(values)
    sel = []
    for i in range(n):
        beaten = 0
        for j in range(n):
            if values[j] > values[i] or (values[j] == values[i] and j < i):
                beaten += 1
        if beaten < k:
            sel.append(i)
    return sel


def _count_round_up(x):
    return int(math.ceil(x - 1e-9))


def _count_round_down(x):
    return int(math.floor(x + 1e-9))


def brute_isa_head(Q, K, V, L_src, L_ctx, b, alpha_s, alpha_f, alpha_ns,
                   enumerate_ctx_subsets=True):
    """Returns dict with O [L, D] and every selection, for one head."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, D = Q.shape
    blocks = _blocks(L_src, L_ctx, b)
    N = len(blocks)
    N_src = sum(1 for (s, _) in blocks if s < L_src)
    N_ctx = N - N_src
    scale = 1.0 / math.sqrt(D)

    Qc = [_mean_loop(Q, s, n) for (s, n) in blocks]
    Kc = [_mean_loop(K, s, n) for (s, n) in blocks]
    Vc = [_mean_loop(V, s, n) for (s, n) in blocks]
    S = [[_dot(Qc[i], Kc[j]) * scale for j in range(N)] for i in range(N)]

    k_ctx = _count_round_up(alpha_s * N_ctx)
    r = [math.fsum(S[i][N_src + c] for i in range(N_src)) for c in range(N_ctx)]
    if enumerate_ctx_subsets:
        best, best_set = -math.inf, None
        for subset in itertools.combinations(range(N_ctx), k_ctx):
            tot = math.fsum(r[c] for c in subset)
            # combinations() yields subsets in lexicographic order, so a strict
            # comparison keeps the lexicographically smallest among equal sums.
            if tot > best:
                best, best_set = tot, subset
        ctx = sorted(best_set) if best_set is not None else []
    else:
        ctx = _rank_select(r, k_ctx)
    J = list(range(N_src)) + [N_src + c for c in ctx]
    N_kv = len(J)

    M = []
    for i in range(N):
        row = [S[i][j] for j in range(N_src)]
        mx = max(row)
        e = [math.exp(x - mx) for x in row]
        z = math.fsum(e)
        p = [x / z for x in e]
        M.append(math.fsum((x - 1.0 / N_src) ** 2 for x in p) / N_src)
    n_flat = _count_round_down(alpha_f * N)
    sharp = _rank_select(M, N - n_flat)
    flat = [i for i in range(N) if i not in sharp]

    k_ns = min(N_kv, _count_round_up(alpha_ns * N_kv))
    E = []
    for i in flat:
        pos = _rank_select([S[i][j] for j in J], k_ns)
        E.append(sorted(J[p] for p in pos))

    O = np.zeros((L, D))
    tok_block = np.empty(L, dtype=np.int64)
    for bi, (s, n) in enumerate(blocks):
        tok_block[s:s + n] = bi
    Kc_a = np.asarray(Kc)
    Vc_a = np.asarray(Vc)
    for t in range(L):
        i = int(tok_block[t])
        logit_parts, value_parts = [], []
        exact_blocks = J if i in sharp else E[flat.index(i)]
        for j in J:
            s, n = blocks[j]
            if j in exact_blocks:
                logit_parts.append(K[s:s + n] @ Q[t] * scale)
                value_parts.append(V[s:s + n])
            else:
                # one pooled term carrying the weight of the block's n tokens
                logit_parts.append(np.array([Kc_a[j] @ Q[t] * scale + math.log(n)]))
                value_parts.append(Vc_a[j][None, :])
        x = np.concatenate(logit_parts)
        w = np.exp(x - x.max())
        O[t] = (w @ np.concatenate(value_parts)) / w.sum()
    return dict(O=O, ctx_idx=np.array(ctx, dtype=np.int64), sharp_idx=np.array(sharp, dtype=np.int64),
                flat_idx=np.array(flat, dtype=np.int64),
                flat_exact_idx=np.array(E, dtype=np.int64).reshape(len(flat), k_ns),
                r=np.array(r), M=np.array(M), S=np.array(S))
