"""Pins for the oracle's backward pass (reading R12: gradients with the
selections held fixed): the special cases that reduce to torch autograd of
library attention, central finite differences of the oracle's own forward,
closed-form sums, and the RoPE transpose written with complex numbers."""
import math

import numpy as np
import pytest
import torch

from oracle import isa_oracle as O


def _rand(seed, L, D, n=4):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((L, D)) for _ in range(n)]


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).requires_grad_(True)


def _selections(Q, K, V, plan):
    r = O.isa_head(Q, K, V, plan, compute_output=False)
    return dict(ctx_idx=r.ctx_idx, sharp_idx=r.sharp_idx, flat_idx=r.flat_idx,
                flat_exact_idx=r.flat_exact_idx)


@pytest.mark.parametrize("L_src,L_ctx,b,D", [(150, 90, 32, 16), (256, 0, 64, 8), (97, 131, 32, 8)])
def test_backward_dense_case_equals_torch_autograd(L_src, L_ctx, b, D):
    """alpha_s = 1, alpha_f = 0: ISA is dense attention, so its gradients
    are those of CPU fp64 scaled_dot_product_attention."""
    plan = O.make_plan(L_src, L_ctx, b, 1.0, 0.0, 0.25)
    Q, K, V, dO = _rand(1, L_src + L_ctx, D)
    gq, gk, gv = O.isa_head_backward(Q, K, V, dO, plan)
    q, k, v = _t(Q), _t(K), _t(V)
    out = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0]
    out.backward(torch.from_numpy(dO))
    for a, t in ((gq, q), (gk, k), (gv, v)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_pure_taylor_equals_autograd_through_pooling():
    """alpha_s = 1, alpha_f = 1, alpha_ns = 0: every token attends the pooled
    keys with logit offset log n_j; torch autograd through the block means
    (torch.mean) and SDPA with that additive mask gives the gradients."""
    L_src, L_ctx, b, D = 200, 170, 32, 16
    plan = O.make_plan(L_src, L_ctx, b, 1.0, 1.0, 0.0)
    Q, K, V, dO = _rand(2, L_src + L_ctx, D)
    gq, gk, gv = O.isa_head_backward(Q, K, V, dO, plan)
    q, k, v = _t(Q), _t(K), _t(V)
    kc = torch.stack([k[s:s + n].mean(0) for s, n in zip(plan.starts, plan.counts)])
    vc = torch.stack([v[s:s + n].mean(0) for s, n in zip(plan.starts, plan.counts)])
    mask = torch.log(torch.tensor(plan.counts, dtype=torch.float64))[None, :].expand(q.shape[0], -1)
    out = torch.nn.functional.scaled_dot_product_attention(q[None], kc[None], vc[None], attn_mask=mask[None])[0]
    out.backward(torch.from_numpy(dO))
    for a, t in ((gq, q), (gk, k), (gv, v)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("gamma", [0.0, 0.7])
@pytest.mark.parametrize("L_src,L_ctx,b,D,a_s,a_f,a_ns,seed", [
    (200, 170, 32, 16, 0.5, 0.5, 0.3, 3),
    (130, 200, 32, 8, 0.25, 0.75, 0.1, 4),
    (64 * 5 + 17, 64 * 4 + 3, 64, 8, 0.5, 0.4, 0.2, 5),
])
def test_backward_matches_central_differences(L_src, L_ctx, b, D, a_s, a_f, a_ns, seed, gamma):
    """<grad, h> equals the central difference of sum(dO * O) along a random
    direction h of (Q, K, V), selections held at those of the unperturbed
    inputs; covers sharp and flat blocks, pruned context blocks, partial
    tail blocks and the residual."""
    plan = O.make_plan(L_src, L_ctx, b, a_s, a_f, a_ns)
    assert plan.n_sharp and plan.n_flat and 0 < plan.k_ns < plan.N_kv and plan.k_ctx < plan.N_ctx
    L = L_src + L_ctx
    Q, K, V, dO = _rand(seed, L, D)
    hQ, hK, hV = _rand(seed + 100, L, D, 3)
    sel = _selections(Q, K, V, plan)
    gq, gk, gv = O.isa_head_backward(Q, K, V, dO, plan, selections=sel, gamma=gamma)

    def f(t):
        r = O.isa_head(Q + t * hQ, K + t * hK, V + t * hV, plan, selections=sel, gamma=gamma)
        return float((dO * r.O).sum())

    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = float((gq * hQ).sum() + (gk * hK).sum() + (gv * hV).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)
    # each input on its own too (a slip in one gradient cannot hide behind another)
    for name, h, g in (("Q", hQ, gq), ("K", hK, gk), ("V", hV, gv)):
        def f1(t):
            args = dict(Q=Q, K=K, V=V)
            args[name] = args[name] + t * h
            r = O.isa_head(args["Q"], args["K"], args["V"], plan, selections=sel, gamma=gamma)
            return float((dO * r.O).sum())
        fd1 = (f1(eps) - f1(-eps)) / (2 * eps)
        an1 = float((g * h).sum())
        assert abs(fd1 - an1) <= 1e-6 * max(1.0, abs(an1)), (name, fd1, an1)


@pytest.mark.parametrize("gamma", [0.0, -0.4])
def test_backward_closed_form_sums(gamma):
    """Every softmax row sums to one, so the value gradients add up to
    (1 + gamma) times the summed output gradient; adding one vector to every
    key shifts each row's logits by a constant, so the key gradients add up
    to zero."""
    plan = O.make_plan(300, 260, 32, 0.5, 0.5, 0.2)
    Q, K, V, dO = _rand(6, 560, 16)
    gq, gk, gv = O.isa_head_backward(Q, K, V, dO, plan, gamma=gamma)
    np.testing.assert_allclose(gv.sum(axis=0), (1 + gamma) * dO.sum(axis=0), rtol=0, atol=1e-9)
    np.testing.assert_allclose(gk.sum(axis=0), 0.0, rtol=0, atol=1e-9)
    # pruned context blocks receive no gradient at all
    sel = _selections(Q, K, V, plan)
    J = set(O.kept_blocks(sel["ctx_idx"], plan).tolist())
    for j in range(plan.N):
        if j not in J:
            s, n = plan.starts[j], plan.counts[j]
            if gamma == 0.0:
                assert not gk[s:s + n].any() and not gv[s:s + n].any()


def test_rope_backward_is_the_conjugate_rotation():
    """Written with complex numbers: the forward multiplies each pair
    x + iy by c + is (the fp32 table values), so the gradient multiplies by
    c - is; and it undoes the unrounded forward rotation to within the fp32
    table's |c + is| - 1."""
    L_src, L_ctx, D, base = 50, 40, 16, 10000.0
    rng = np.random.default_rng(7)
    Y = rng.standard_normal((L_src + L_ctx, D))
    c, s = O.rope_tables(O.rope_positions(L_src, L_ctx), D, base)
    w = c.astype(np.float64) + 1j * s.astype(np.float64)
    yz = Y[:, 0::2] + 1j * Y[:, 1::2]
    g = O.rope_backward(Y, L_src, L_ctx, base)
    gz = yz * np.conj(w)
    np.testing.assert_allclose(g[:, 0::2], gz.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(g[:, 1::2], gz.imag, rtol=0, atol=1e-14)
    X = rng.standard_normal((L_src + L_ctx, D))
    xz = (X[:, 0::2] + 1j * X[:, 1::2]) * w
    R = np.empty_like(X)
    R[:, 0::2], R[:, 1::2] = xz.real, xz.imag
    np.testing.assert_allclose(O.rope_backward(R, L_src, L_ctx, base), X, rtol=0, atol=1e-6)


def test_row_sampled_dq_matches_full_backward():
    """The row-by-row dQ (for sampling large shapes) equals the full
    backward's rows, sharp and flat alike."""
    plan = O.make_plan(200, 170, 32, 0.5, 0.5, 0.3)
    Q, K, V, dO = _rand(8, 370, 16)
    gq, _, _ = O.isa_head_backward(Q, K, V, dO, plan)
    rows = np.array([0, 5, 63, 64, 150, 199, 200, 250, 369])
    np.testing.assert_allclose(O.isa_head_dq_rows(Q, K, V, dO, plan, rows), gq[rows], rtol=1e-10, atol=1e-12)
