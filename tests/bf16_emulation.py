"""A CPU model of the bf16 storage of the HIP path's intermediates.

TEST INFRASTRUCTURE ONLY: it derives the tolerances of the GPU parity tests
whose inputs cannot meet the plain bf16 bound.  It is the oracle's arithmetic
(float64, the same steps) with a round-to-nearest-even bf16 rounding inserted
wherever the HIP path stores a tensor in bf16 between kernels or feeds one to
a bf16 matrix core:

* prefill: c_q (the down-projection output) and its RMS-normalised value,
  c_kv, k_pe (before and after RoPE), q_nope, q_pe (before and after RoPE),
  k_nope, v, the softmax probabilities fed to the P V product, o, and y;
* absorbed decode: c_q and its normalised value, q_nope, q_pe (before and
  after RoPE), the new latent row (before and after RoPE), q_lat, the
  probabilities fed to the P C product, o_lat, o and y.

Everything else is exact (float64): the products' accumulation, the softmax
max and sum.  So the model's error against the oracle is the error that bf16
storage alone forces on a given input, whatever the kernels do; a kernel
that meets it within a small factor adds little error of its own.
"""

from __future__ import annotations

import numpy as np

import oracle as orc
from synth_inputs import round_bf16


def _round(a):
    return round_bf16(np.asarray(a, dtype=np.float64).astype(np.float32)).astype(np.float64)


def _keep(a):
    return np.asarray(a, dtype=np.float64)


def _attention_bf16_p(q, k, v, scale, _r, q_pos=None):
    """Causal softmax attention with the probabilities rounded to bf16 for
    the P V product (the normaliser is the exact sum)."""
    sq, sk = q.shape[0], k.shape[0]
    if q_pos is None:
        q_pos = np.arange(sq)
    s = scale * (q @ k.T)
    s = np.where(np.arange(sk)[None, :] > np.asarray(q_pos)[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return (_r(p) @ v) / p.sum(axis=-1, keepdims=True)


def bound(strict: float, modelled: float) -> float:
    """Tolerance for an input whose bf16 storage alone forces an error of
    ``modelled``: the strict bound, or 1.6 x the modelled error where that is
    larger (the HIP path's own roundings fall differently from the model's,
    so its error scatters around the modelled one)."""
    return max(strict, 1.6 * modelled)


def prefill_bf16(cfg: orc.Cfg, w: dict, x, rounding: bool = True):
    """y [B, S, D] of the prefill with bf16 storage of the intermediates
    (rounding=False: no rounding at all, i.e. the oracle's result)."""
    _r = _round if rounding else _keep
    x = np.asarray(x, dtype=np.float64)
    B, S, _ = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    pos = np.arange(S)
    c_q = _r(x @ f["w_down_q"].T)
    c_qn = _r(orc.rmsnorm(c_q, f["q_norm"], cfg.rms_norm_eps))
    q_nope = _r(c_qn @ f["w_up_q"].T).reshape(B, S, H, dn)
    q_pe = _r(c_qn @ f["w_qr"].T).reshape(B, S, H, dr)
    c_kv = _r(x @ f["w_down_kv"].T)
    k_pe = _r(x @ f["w_kr"].T)
    q_pe = _r(np.stack([orc.apply_rope(q_pe[b], pos, cfg) for b in range(B)]))
    k_pe = _r(np.stack([orc.apply_rope(k_pe[b], pos, cfg) for b in range(B)]))
    k_nope = _r(c_kv @ f["w_up_k"].T).reshape(B, S, H, dn)
    v = _r(c_kv @ f["w_up_v"].T).reshape(B, S, H, dv)
    scale = orc.softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            q = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            k = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = _attention_bf16_p(q, k, v[b, :, h], scale, _r)
    o = _r(o).reshape(B, S, H * dv)
    return _r(o @ f["wo"].T)


def decode_absorbed_bf16(cfg: orc.Cfg, w: dict, x, cache, lens, rounding: bool = True):
    """y [B, D] of one absorbed decode step with bf16 storage of the
    intermediates (cache rows are bf16 values already; rounding=False: the
    oracle's result)."""
    _r = _round if rounding else _keep
    x = np.asarray(x, dtype=np.float64)
    B = x.shape[0]
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    r = cfg.kv_lora_rank
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    wuk = f["w_up_k"].reshape(H, dn, r)
    wuv = f["w_up_v"].reshape(H, dv, r)
    scale = orc.softmax_scale(cfg)
    y = np.empty((B, cfg.hidden_size))
    for b in range(B):
        L = int(lens[b])
        xb = x[b]
        c_qn = _r(orc.rmsnorm(_r(xb @ f["w_down_q"].T), f["q_norm"], cfg.rms_norm_eps))
        q_nope = _r(c_qn @ f["w_up_q"].T).reshape(H, dn)
        q_pe = _r(orc.apply_rope(_r(c_qn @ f["w_qr"].T).reshape(1, H, dr), [L], cfg)[0])
        c_new = _r(xb @ f["w_down_kv"].T)
        k_new = _r(orc.apply_rope(_r(xb @ f["w_kr"].T)[None, :], [L], cfg)[0])
        rows = np.concatenate([np.asarray(cache[b, :L], dtype=np.float64),
                               np.concatenate([c_new, k_new])[None]], axis=0)
        c, kp = rows[:, :r], rows[:, r:]
        q_lat = _r(np.einsum("hd,hdr->hr", q_nope, wuk))
        s = scale * (q_lat @ c.T + q_pe @ kp.T)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        o_lat = _r((_r(p) @ c) / p.sum(axis=-1, keepdims=True))
        o = _r(np.einsum("hvr,hr->hv", wuv, o_lat))
        y[b] = _r(o.reshape(-1) @ f["wo"].T)
    return y


def prefill_fp8_bf16(cfg: orc.Cfg, w: dict, x):
    """y [B, S, D] of the FP8 prefill (oracle.fp8_oracle.mla_prefill_fp8)
    with bf16 storage of the intermediates the HIP path keeps in bf16 (the
    projection outputs, RMSNorm(c_q), post-RoPE q_pe / k_pe, the softmax
    probabilities, o, y); each projection input is quantised from those
    stored values, as on the device."""
    from oracle import fp8_oracle as fo
    _r = _round
    x = np.asarray(x, dtype=np.float64)
    B, S, D = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items() if v is not None}
    xf = x.reshape(B * S, D)
    c_q = _r(fo.quantized_product(xf, f["w_down_q"]))
    c_kv = _r(fo.quantized_product(xf, f["w_down_kv"]))
    k_pe = _r(fo.quantized_product(xf, f["w_kr"]))
    c_qn = _r(orc.rmsnorm(c_q, f["q_norm"], cfg.rms_norm_eps))
    if "kv_norm" in f:
        c_kv = _r(orc.rmsnorm(c_kv, f["kv_norm"], cfg.rms_norm_eps))
    q_nope = _r(fo.quantized_product(c_qn, f["w_up_q"])).reshape(B, S, H, dn)
    q_pe = _r(fo.quantized_product(c_qn, f["w_qr"])).reshape(B, S, H, dr)
    k_nope = _r(fo.quantized_product(c_kv, f["w_up_k"])).reshape(B, S, H, dn)
    v = _r(fo.quantized_product(c_kv, f["w_up_v"])).reshape(B, S, H, dv)
    pos = np.arange(S)
    q_pe = _r(np.stack([orc.apply_rope(q_pe[b], pos, cfg) for b in range(B)]))
    k_pe = _r(np.stack([orc.apply_rope(k_pe.reshape(B, S, dr)[b], pos, cfg) for b in range(B)]))
    scale = orc.softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            q = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            k = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = _attention_bf16_p(q, k, v[b, :, h], scale, _r)
    o = _r(o).reshape(B * S, H * dv)
    return _r(fo.quantized_product(o, f["wo"])).reshape(B, S, D)


def prefill_fp8_bf16_rows(cfg: orc.Cfg, w: dict, x, rows, batch: int = 0):
    """Rows ``rows`` of :func:`prefill_fp8_bf16` (keys and values head by
    head, queries only for those rows), for V3 sizes."""
    from oracle import fp8_oracle as fo
    _r = _round
    xb = np.asarray(x[batch], dtype=np.float64)
    S, D = xb.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    rows = np.asarray(rows, dtype=np.int64)
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items() if v is not None}
    pos = np.arange(S)
    xq = fo.qdq_act(xb)
    c_kv = _r(xq @ fo.qdq_weight(f["w_down_kv"]).T)
    if "kv_norm" in f:
        c_kv = _r(orc.rmsnorm(c_kv, f["kv_norm"], cfg.rms_norm_eps))
    k_pe = _r(orc.apply_rope(_r(xq @ fo.qdq_weight(f["w_kr"]).T), pos, cfg))
    c_qn = _r(orc.rmsnorm(_r(xq[rows] @ fo.qdq_weight(f["w_down_q"]).T), f["q_norm"], cfg.rms_norm_eps))
    q_nope = _r(fo.quantized_product(c_qn, f["w_up_q"])).reshape(len(rows), H, dn)
    q_pe = _r(orc.apply_rope(_r(fo.quantized_product(c_qn, f["w_qr"])).reshape(len(rows), H, dr), rows, cfg))
    kmax = int(rows.max()) + 1
    ca = fo.qdq_act(c_kv[:kmax])
    wuk = fo.qdq_weight(f["w_up_k"])
    wuv = fo.qdq_weight(f["w_up_v"])
    scale = orc.softmax_scale(cfg)
    o = np.empty((len(rows), H, dv))
    for h in range(H):
        k = np.concatenate([_r(ca @ wuk[h * dn:(h + 1) * dn].T), k_pe[:kmax]], axis=-1)
        v = _r(ca @ wuv[h * dv:(h + 1) * dv].T)
        q = np.concatenate([q_nope[:, h], q_pe[:, h]], axis=-1)
        o[:, h] = _attention_bf16_p(q, k, v, scale, _r, q_pos=rows)
    return _r(fo.quantized_product(_r(o).reshape(len(rows), H * dv), f["wo"]))


def mla_backward_bf16(cfg: orc.Cfg, w: dict, x, dy, rounding: bool = True):
    """The MLA backward oracle's chain rule (oracle.mla_backward_oracle) with
    bf16 storage wherever the HIP path stores bf16: the forward intermediates
    (c_q before and after its norm, c_kv, k_pe, q, k_nope, v, o), do, the
    attention backward's dq / dk / dv, the shared key's summed gradient and
    both RoPE backwards, dc_qn, dc_kv, dc_q, and every output (dx and the
    weight gradients; the gains' gradients stay fp32).  Sums run exactly."""
    from oracle.attn_backward_oracle import causal_attention_backward, rmsnorm_backward
    from oracle.mla_backward_oracle import rope_backward
    _r = _round if rounding else _keep
    x, dy = np.asarray(x, dtype=np.float64), np.asarray(dy, dtype=np.float64)
    B, S, D = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items() if v is not None}
    eps = cfg.rms_norm_eps
    pos = np.arange(S)
    M = B * S
    xf = x.reshape(M, D)
    c_q = _r(xf @ f["w_down_q"].T)
    c_qn = _r(orc.rmsnorm(c_q, f["q_norm"], eps))
    c_kv_raw = _r(xf @ f["w_down_kv"].T)
    c_kv = _r(orc.rmsnorm(c_kv_raw, f["kv_norm"], eps)) if "kv_norm" in f else c_kv_raw
    k_pe = _r(np.stack([orc.apply_rope(_r(xf @ f["w_kr"].T).reshape(B, S, dr)[b], pos, cfg) for b in range(B)]))
    q_nope = _r(c_qn @ f["w_up_q"].T).reshape(B, S, H, dn)
    q_pe = _r(np.stack([orc.apply_rope(_r(c_qn @ f["w_qr"].T).reshape(B, S, H, dr)[b], pos, cfg)
                        for b in range(B)]))
    k_nope = _r(c_kv @ f["w_up_k"].T).reshape(B, S, H, dn)
    v = _r(c_kv @ f["w_up_v"].T).reshape(B, S, H, dv)
    scale = orc.softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    qh = np.empty((B, H, S, dn + dr))
    kh = np.empty((B, H, S, dn + dr))
    for b in range(B):
        for h in range(H):
            qh[b, h] = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            kh[b, h] = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = _attention_bf16_p(qh[b, h], kh[b, h], v[b, :, h], scale, _r)
    of = _r(o).reshape(M, H * dv)
    g = {}
    dyf = dy.reshape(M, D)
    g["wo"] = _r(dyf.T @ of)
    do = _r(dyf @ f["wo"]).reshape(B, S, H, dv)
    dq_nope = np.empty((B, S, H, dn))
    dq_pe = np.empty((B, S, H, dr))
    dk_nope = np.empty((B, S, H, dn))
    dk_pe = np.zeros((B, S, dr))
    dvv = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            dqh, dkh, dvh = (_r(t) for t in causal_attention_backward(qh[b, h], kh[b, h], v[b, :, h],
                                                                      do[b, :, h], scale,
                                                                      o=of.reshape(B, S, H, dv)[b, :, h]))
            dq_nope[b, :, h], dq_pe[b, :, h] = dqh[:, :dn], dqh[:, dn:]
            dk_nope[b, :, h] = dkh[:, :dn]
            dk_pe[b] += dkh[:, dn:]
            dvv[b, :, h] = dvh
    dk_pe = _r(dk_pe)
    dq_pe_raw = _r(np.stack([rope_backward(dq_pe[b], pos, cfg) for b in range(B)])).reshape(M, H * dr)
    dk_pe_raw = _r(np.stack([rope_backward(dk_pe[b], pos, cfg) for b in range(B)])).reshape(M, dr)
    dq_nope = dq_nope.reshape(M, H * dn)
    dk_nope = dk_nope.reshape(M, H * dn)
    dvv = dvv.reshape(M, H * dv)
    g["w_up_q"] = _r(dq_nope.T @ c_qn)
    g["w_qr"] = _r(dq_pe_raw.T @ c_qn)
    dc_qn = _r(dq_nope @ f["w_up_q"] + dq_pe_raw @ f["w_qr"])
    g["w_up_k"] = _r(dk_nope.T @ c_kv)
    g["w_up_v"] = _r(dvv.T @ c_kv)
    dc_kv = _r(dk_nope @ f["w_up_k"] + dvv @ f["w_up_v"])
    if "kv_norm" in f:
        dc_kv_raw, g["kv_norm"] = rmsnorm_backward(c_kv_raw, f["kv_norm"], dc_kv, eps)
        dc_kv_raw = _r(dc_kv_raw)
    else:
        dc_kv_raw = dc_kv
    dc_q, g["q_norm"] = rmsnorm_backward(c_q, f["q_norm"], dc_qn, eps)
    dc_q = _r(dc_q)
    g["w_down_q"] = _r(dc_q.T @ xf)
    g["w_down_kv"] = _r(dc_kv_raw.T @ xf)
    g["w_kr"] = _r(dk_pe_raw.T @ xf)
    dx = _r(dc_q @ f["w_down_q"] + dc_kv_raw @ f["w_down_kv"] + dk_pe_raw @ f["w_kr"])
    return dx.reshape(B, S, D), g
