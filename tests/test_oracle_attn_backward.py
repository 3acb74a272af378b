"""Pins of the attention-backward oracle: finite differences, torch autograd
(float64, an independent implementation) and the softmax shift invariances
(no GPU)."""

import numpy as np
import torch

from oracle import attn_backward_oracle as ab

RNG = np.random.default_rng(31)


def _case(S=7, dqk=5, dv=4):
    return (RNG.standard_normal((S, dqk)), RNG.standard_normal((S, dqk)),
            RNG.standard_normal((S, dv)), RNG.standard_normal((S, dv)))


def test_finite_differences():
    q, k, v, do = _case()
    scale = 0.7
    dq, dk, dv = ab.causal_attention_backward(q, k, v, do, scale)
    loss = lambda q_, k_, v_: float(np.sum(do * ab.attention_forward_heads(q_[None], k_[None], v_[None], scale)[0]))
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * (1 + abs(fd)), (name, idx, fd, g[idx])


def test_matches_torch_autograd():
    q, k, v, do = (RNG.standard_normal((3, 2, 33, d)) for d in (24, 24, 16, 16))
    scale = 24 ** -0.5
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    mask = torch.ones(33, 33, dtype=torch.bool).triu(1)
    p = torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1)
    (p @ tv).backward(torch.tensor(do))
    dq, dk, dv = ab.attention_backward_heads(q, k, v, do, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_shift_invariances():
    # adding one vector to every key leaves each softmax row unchanged, so the
    # key gradients sum to zero; adding one to every value shifts each output
    # row by it, so the value gradients sum to the summed upstream gradient
    q, k, v, do = _case(S=20, dqk=9, dv=6)
    dq, dk, dv = ab.causal_attention_backward(q, k, v, do, 0.4)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_first_query_sees_only_itself():
    # query 0 attends key 0 alone: p = 1, no gradient through its scores
    q, k, v, do = _case(S=6)
    dq, dk, dv = ab.causal_attention_backward(q, k, v, do, 0.9)
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-14)
    # the last key is seen only by the last query
    p_last = ab.causal_attention_probs(q, k, 0.9)[-1, -1]
    np.testing.assert_allclose(dv[-1], p_last * do[-1], rtol=1e-12)


def test_given_output_enters_through_delta_only():
    # handing the exact forward output changes nothing; a perturbed one moves
    # dS by -P * rowsum(dout * perturbation), so dV is unaffected
    q, k, v, do = _case(S=9)
    ref = ab.causal_attention_backward(q, k, v, do, 0.6)
    o = ab.attention_forward_heads(q[None], k[None], v[None], 0.6)[0]
    same = ab.causal_attention_backward(q, k, v, do, 0.6, o=o)
    for a, b in zip(ref, same):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    eps = 1e-3 * RNG.standard_normal(o.shape)
    pert = ab.causal_attention_backward(q, k, v, do, 0.6, o=o + eps)
    np.testing.assert_allclose(pert[2], ref[2], rtol=1e-12, atol=1e-14)
    p = ab.causal_attention_probs(q, k, 0.6)
    shift = np.sum(do * eps, axis=-1, keepdims=True)
    np.testing.assert_allclose(pert[0], ref[0] - 0.6 * (p * shift) @ k, rtol=1e-9, atol=1e-12)


def test_rmsnorm_backward_finite_differences_and_autograd():
    from oracle.mla_oracle import rmsnorm
    x = RNG.standard_normal((4, 12))
    g = 1 + 0.1 * RNG.standard_normal(12)
    dy = RNG.standard_normal((4, 12))
    eps = 1e-6
    dx, dg = ab.rmsnorm_backward(x, g, dy, eps)
    loss = lambda x_, g_: float(np.sum(dy * rmsnorm(x_, g_, eps)))
    h = 1e-6
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (loss(xp, g) - loss(xm, g)) / (2 * h)
        assert abs(fd - dx[idx]) <= 1e-6 * (1 + abs(fd))
    for c in range(12):
        gp, gm = g.copy(), g.copy()
        gp[c] += h
        gm[c] -= h
        fd = (loss(x, gp) - loss(x, gm)) / (2 * h)
        assert abs(fd - dg[c]) <= 1e-6 * (1 + abs(fd))
    tx, tg = torch.tensor(x, requires_grad=True), torch.tensor(g, requires_grad=True)
    torch.nn.functional.rms_norm(tx, (12,), tg, eps).backward(torch.tensor(dy))
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    # scale invariance of the normalisation: x is orthogonal to dx when eps = 0
    dx0, _ = ab.rmsnorm_backward(x, g, dy, 0.0)
    np.testing.assert_allclose(np.sum(dx0 * x, axis=-1), 0.0, atol=1e-10)
