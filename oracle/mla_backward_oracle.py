"""Plain float64 oracle of the MLA backward: every gradient of the prefill.

TEST INFRASTRUCTURE ONLY -- never on the product path.

Source: the forward of "The Evolving Transformer -- DeepSeek V2 & V3",
section 01 "Multi-head Latent Attention (MLA)" (with the readings of
oracle.mla_oracle: RMSNorm on c_q, optional RMSNorm on c_kv, one shared RoPE
key), whose training the "DSV3 Native PyTorch Reference" README checks by
finite differences ("NumPy Oracle" section).  For an upstream gradient dy of
y = MLA(x) the gradients are the chain rule through the forward's steps, in
reverse order, written out one by one:

    y = o W_o^T                 dW_o = dy^T o,     do = dy W_o
    o_h = attn(q_h, k_h, v_h)   (dq_h, dk_h, dv_h) = attention backward
    k_h = [k_nope_h ‖ k_pe]     dk_pe = sum over heads of dk_h's rope part
    q_pe = R(p) q_pe_raw        dq_pe_raw = R(p)^T dq_pe = R(-p) dq_pe
    k_pe = R(p) k_pe_raw        dk_pe_raw = R(-p) dk_pe (the amplitude of
                                YaRN multiplies both)
    q_nope = c_qn W_uq^T        dW_uq = dq_nope^T c_qn, dc_qn += dq_nope W_uq
    q_pe_raw = c_qn W_qr^T      dW_qr = dq_pe_raw^T c_qn, dc_qn += dq_pe_raw W_qr
    k_nope = c_kv W_uk^T        dW_uk = dk_nope^T c_kv, dc_kv += dk_nope W_uk
    v = c_kv W_uv^T             dW_uv = dv^T c_kv, dc_kv += dv W_uv
    c_qn = RMSNorm(c_q) g_q     (dc_q, dg_q) = RMSNorm backward
    c_kv = RMSNorm(c_kv_raw) g_kv (when kv_norm is given; else c_kv = c_kv_raw)
    c_q = x W_dq^T              dW_dq = dc_q^T x, dx += dc_q W_dq
    c_kv_raw = x W_dkv^T        dW_dkv = dc_kv_raw^T x, dx += dc_kv_raw W_dkv
    k_pe_raw = x W_kr^T         dW_kr = dk_pe_raw^T x, dx += dk_pe_raw W_kr

The tests pin the result to central finite differences of <dy, y> in every
parameter and to torch autograd of an independent torch forward.
"""

from __future__ import annotations

import numpy as np

from .attn_backward_oracle import causal_attention_backward, rmsnorm_backward
from .mla_oracle import apply_rope, causal_attention, rmsnorm, softmax_scale


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def rope_backward(g, positions, cfg):
    """Gradient through the RoPE rotation at ``positions``: the transposed
    rotation, i.e. the rotation by the negated angle (times the same YaRN
    amplitude)."""
    return apply_rope(g, -np.asarray(positions), cfg)


def mla_backward(cfg, w: dict, x, dy):
    """Gradients of <dy, MLA(x)> for x [B, S, D] at positions 0..S-1.

    Returns (dx [B, S, D], grads) with grads[name] shaped like w[name] for
    every weight of w (q_norm and, if given, kv_norm included)."""
    x, dy = _f64(x), _f64(dy)
    B, S, D = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    f = {k: _f64(v) for k, v in w.items() if v is not None}
    eps = cfg.rms_norm_eps
    pos = np.arange(S)
    M = B * S
    xf = x.reshape(M, D)

    # forward, keeping what the backward reads
    c_q = xf @ f["w_down_q"].T
    c_qn = rmsnorm(c_q, f["q_norm"], eps)
    c_kv_raw = xf @ f["w_down_kv"].T
    c_kv = rmsnorm(c_kv_raw, f["kv_norm"], eps) if "kv_norm" in f else c_kv_raw
    k_pe = np.stack([apply_rope((xf @ f["w_kr"].T).reshape(B, S, dr)[b], pos, cfg) for b in range(B)])
    q_nope = (c_qn @ f["w_up_q"].T).reshape(B, S, H, dn)
    q_pe_raw = (c_qn @ f["w_qr"].T).reshape(B, S, H, dr)
    q_pe = np.stack([apply_rope(q_pe_raw[b], pos, cfg) for b in range(B)])
    k_nope = (c_kv @ f["w_up_k"].T).reshape(B, S, H, dn)
    v = (c_kv @ f["w_up_v"].T).reshape(B, S, H, dv)
    scale = softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    qh = np.empty((B, H, S, dn + dr))
    kh = np.empty((B, H, S, dn + dr))
    for b in range(B):
        for h in range(H):
            qh[b, h] = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            kh[b, h] = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = causal_attention(qh[b, h], kh[b, h], v[b, :, h], scale)
    of = o.reshape(M, H * dv)

    # backward
    g = {}
    dyf = dy.reshape(M, D)
    g["wo"] = dyf.T @ of
    do = (dyf @ f["wo"]).reshape(B, S, H, dv)
    dq_nope = np.empty((B, S, H, dn))
    dq_pe = np.empty((B, S, H, dr))
    dk_nope = np.empty((B, S, H, dn))
    dk_pe = np.zeros((B, S, dr))
    dvv = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            dqh, dkh, dvh = causal_attention_backward(qh[b, h], kh[b, h], v[b, :, h], do[b, :, h], scale)
            dq_nope[b, :, h], dq_pe[b, :, h] = dqh[:, :dn], dqh[:, dn:]
            dk_nope[b, :, h] = dkh[:, :dn]
            dk_pe[b] += dkh[:, dn:]  # the RoPE key is shared by every head
            dvv[b, :, h] = dvh
    dq_pe_raw = np.stack([rope_backward(dq_pe[b], pos, cfg) for b in range(B)]).reshape(M, H * dr)
    dk_pe_raw = np.stack([rope_backward(dk_pe[b], pos, cfg) for b in range(B)]).reshape(M, dr)
    dq_nope = dq_nope.reshape(M, H * dn)
    dk_nope = dk_nope.reshape(M, H * dn)
    dvv = dvv.reshape(M, H * dv)
    g["w_up_q"] = dq_nope.T @ c_qn
    g["w_qr"] = dq_pe_raw.T @ c_qn
    dc_qn = dq_nope @ f["w_up_q"] + dq_pe_raw @ f["w_qr"]
    g["w_up_k"] = dk_nope.T @ c_kv
    g["w_up_v"] = dvv.T @ c_kv
    dc_kv = dk_nope @ f["w_up_k"] + dvv @ f["w_up_v"]
    if "kv_norm" in f:
        dc_kv_raw, g["kv_norm"] = rmsnorm_backward(c_kv_raw, f["kv_norm"], dc_kv, eps)
    else:
        dc_kv_raw = dc_kv
    dc_q, g["q_norm"] = rmsnorm_backward(c_q, f["q_norm"], dc_qn, eps)
    g["w_down_q"] = dc_q.T @ xf
    g["w_down_kv"] = dc_kv_raw.T @ xf
    g["w_kr"] = dk_pe_raw.T @ xf
    dx = dc_q @ f["w_down_q"] + dc_kv_raw @ f["w_down_kv"] + dk_pe_raw @ f["w_kr"]
    return dx.reshape(B, S, D), g
