"""Plain float64 oracle of the causal attention backward (dQ, dK, dV).

TEST INFRASTRUCTURE ONLY -- never on the product path.

Source: "The Evolving Transformer -- DeepSeek V2 & V3", section 01
"Multi-head Latent Attention (MLA)": the forward whose gradients these are,
per head P = softmax(scale Q K^T with the causal tril mask), O = P V.  The
first page's reference ("dsv3-native-reference" README) trains the model and
checks its gradients by finite differences; the backward is the training
half of the pages.

The gradients are the chain rule through those three steps, written out:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(dO * O))     (softmax backward; masked entries 0)
    dQ = scale dS K,   dK = scale dS^T Q

The tests pin them against central finite differences, against torch
autograd in float64, and against the shift invariances of the softmax.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import causal_attention


def causal_attention_probs(q, k, scale):
    """P [Sq, Sk] of one head (causal tril mask, query r at position r)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T)
    mask = np.arange(k.shape[0])[None, :] > np.arange(q.shape[0])[:, None]
    s = np.where(mask, -np.inf, s)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    return p / np.sum(p, axis=-1, keepdims=True)


def causal_attention_backward(q, k, v, dout, scale, o=None):
    """(dq, dk, dv) of one head for the upstream gradient dout [Sq, dv].

    o is the forward output the backward is handed (the stored O, which
    enters through rowsum(dO * O)); by default the exact P V."""
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    p = causal_attention_probs(q, k, scale)
    o = p @ v if o is None else np.asarray(o, dtype=np.float64)
    dv = p.T @ dout
    dp = dout @ v.T
    delta = np.sum(dout * o, axis=-1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward_heads(q, k, v, dout, scale, o=None):
    """Batched over leading axes: q, k [..., S, dqk], v, dout [..., S, dv];
    o (optional) the stored forward output [..., S, dv]."""
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    lead = q.shape[:-2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for idx in np.ndindex(*lead):
        dq[idx], dk[idx], dv[idx] = causal_attention_backward(q[idx], k[idx], v[idx], dout[idx], scale,
                                                              None if o is None else o[idx])
    return dq, dk, dv


def attention_forward_heads(q, k, v, scale):
    """Forward O of every head (the same causal attention the prefill uses)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    o = np.zeros(q.shape[:-1] + (v.shape[-1],))
    for idx in np.ndindex(*q.shape[:-2]):
        o[idx] = causal_attention(q[idx], k[idx], v[idx], scale)
    return o


def rmsnorm_backward(x, g, dy, eps):
    """(dx, dg) of y = x * (mean(x^2) + eps)^-1/2 * g over the last axis (the
    RMSNorm on c_q of the MLA module), float64:
    dx = r (g dy) - x r^3 mean(x g dy), dg = sum over rows of dy x r."""
    x, g, dy = (np.asarray(a, dtype=np.float64) for a in (x, g, dy))
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gdy = g * dy
    dx = r * gdy - x * r ** 3 * np.mean(x * gdy, axis=-1, keepdims=True)
    dg = np.sum((dy * x * r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dg
