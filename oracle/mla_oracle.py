"""Plain float64 oracle of the DeepSeek-V3 MLA forward (prefill, decode, RoPE).

TEST INFRASTRUCTURE ONLY -- never on the product path.  Slow and obvious on
purpose: every step is the plain definition, written with NumPy float64
matrix products and nothing fused, blocked or reordered.

Sources (pages, by title and section):

* "The Evolving Transformer -- DeepSeek V2 & V3", section 01 "Multi-head
  Latent Attention (MLA)": the ``MultiHeadLatentAttention`` module (the
  projections w_down_kv, w_up_k, w_up_v, w_kr, w_down_q, w_up_q, w_qr, wo;
  K = cat(K_nope, K_rope), Q = cat(Q_nope, Q_rope), V from the nope width only;
  scores Q K^T / sqrt(dk) with the causal tril mask, softmax, times V, heads
  concatenated head-major, then wo) and the cache formula under it (c_kv is
  what is cached; K_i and V_i are up-projections of c_kv).
* Same page, section 05 "Assemble DeepSeek (V3)": RoPE is sized by the rope
  head dim only; the mask is a full tril (no sliding window).
* "DeepSeek-V3 Decoupled Implementation" (README), "Architecture" list and
  "Key Dimensions (671B variant)" table: 512-dim latent, decoupled 64-dim RoPE
  stream, YaRN factor 40 to 163,840 tokens, rms_norm_eps 1e-6 and the V3 sizes.
* "[DeepSeek-V3] Different rotary embedding implementation between DeepSeek-AI
  and Transformers" (transformers issue 39687): the complex (interleaved-pair)
  and the Eleuther (rotate-half) RoPE formulations give different results on
  the same q_pe/k_pe and agree once the q_pe/k_pe columns (equivalently the
  rows of the weights producing them) are permuted by the even/odd
  de-interleave.

Readings where the pages are silent (each is listed in the design doc):

* RMSNorm is x * (mean(x^2) + eps)^-1/2 * g, applied to c_q before both w_up_q
  and w_qr; there is no norm on c_kv (optional kv_norm gains, for
  checkpoints that normalise the latent, apply the same norm to c_kv).
* The RoPE key k_pe is one shared d_r vector per token, broadcast to all heads.
* The softmax scale is (d_nope + d_rope)^-1/2, also in decode; with YaRN it is
  multiplied by mscale(factor, mscale_all_dim)^2.
* inv_freq_i = theta^(-2i/d_r); pair i of both conventions uses inv_freq_i;
  the rotation is by +angle; positions start at 0; angles are float64.
* YaRN uses the index-space linear ramp between the correction dims of
  beta_fast and beta_slow; the pages fix only its reductions, and the tests
  pin the rest to the DeepSeek-V3 code of `transformers` that the RoPE page
  names.
* Decode: the new token sits at position L_b (= rows already cached) and
  attends to cache rows 0..L_b including itself; the cache holds c_kv and the
  post-RoPE k_pe, in the layout of the convention in use.

Weights are ``nn.Linear`` matrices: shape [out, in], y = x W^T, no bias.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HALF_SPLIT = "half_split"
INTERLEAVED = "interleaved"


@dataclass
class Cfg:
    """MLA shape and RoPE settings, with DeepSeek-V3 config field names."""

    hidden_size: int
    num_attention_heads: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    rms_norm_eps: float = 1e-6
    rope_theta: float = 10000.0
    rope_convention: str = HALF_SPLIT
    # YaRN; factor 1 means plain RoPE
    rope_factor: float = 1.0
    original_max_position_embeddings: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 1.0
    softmax_scale_override: Optional[float] = None
    extra: dict = field(default_factory=dict)


# ---------------------------------------------------------------- RoPE ----

def rope_inv_freq(rope_dim: int, theta: float) -> np.ndarray:
    """inv_freq_i = theta^(-2i/d_r), i = 0..d_r/2-1, float64."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / rope_dim)


def _yarn_correction_dim(num_rotations: float, dim: int, base: float,
                         original_max: int) -> float:
    # the (fractional) pair index whose wavelength fits num_rotations times
    # into the original context: original_max * inv_freq_i / (2 pi) = rot
    return (dim * math.log(original_max / (num_rotations * 2.0 * math.pi))) / (
        2.0 * math.log(base))


def yarn_correction_range(dim: int, base: float, original_max: int,
                          beta_fast: float, beta_slow: float):
    """(low, high) pair indices of the YaRN ramp, clamped to [0, dim-1]."""
    low = math.floor(_yarn_correction_dim(beta_fast, dim, base, original_max))
    high = math.ceil(_yarn_correction_dim(beta_slow, dim, base, original_max))
    return max(low, 0), min(high, dim - 1)


def yarn_inv_freq(rope_dim: int, theta: float, factor: float,
                  original_max: int, beta_fast: float,
                  beta_slow: float) -> np.ndarray:
    """YaRN frequencies: keep high-frequency pairs, divide low-frequency
    pairs by ``factor``, linear ramp in pair index in between."""
    base = rope_inv_freq(rope_dim, theta)
    if factor == 1.0:
        return base
    low, high = yarn_correction_range(rope_dim, theta, original_max,
                                      beta_fast, beta_slow)
    hi = float(high) if high != low else float(high) + 0.001
    idx = np.arange(rope_dim // 2, dtype=np.float64)
    ramp = np.clip((idx - low) / (hi - low), 0.0, 1.0)
    return base * (1.0 - ramp) + (base / factor) * ramp


def yarn_mscale(scale: float, mscale: float) -> float:
    """Attention temperature factor of YaRN: 0.1 m ln(s) + 1 for s > 1."""
    if scale <= 1.0:
        return 1.0
    return 0.1 * mscale * math.log(scale) + 1.0


def cfg_inv_freq(cfg: Cfg) -> np.ndarray:
    return yarn_inv_freq(cfg.qk_rope_head_dim, cfg.rope_theta, cfg.rope_factor,
                         cfg.original_max_position_embeddings, cfg.beta_fast,
                         cfg.beta_slow)


def cfg_cos_sin_scale(cfg: Cfg) -> float:
    return yarn_mscale(cfg.rope_factor, cfg.mscale) / yarn_mscale(
        cfg.rope_factor, cfg.mscale_all_dim)


def rope_cos_sin(positions, inv_freq, amp: float = 1.0):
    """cos/sin of angle p * inv_freq_i in float64: shapes [T, d_r/2]."""
    p = np.asarray(positions, dtype=np.float64)
    ang = p[:, None] * inv_freq[None, :]
    return np.cos(ang) * amp, np.sin(ang) * amp


def rope_half_split(x, cos, sin):
    """Rotate-half RoPE: pair (i, i + d/2) turned by angle_i.

    x: [T, ..., d]; cos/sin: [T, d/2] (broadcast over the middle axes)."""
    d = x.shape[-1]
    h = d // 2
    shp = (cos.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = cos.reshape(shp)
    s = sin.reshape(shp)
    x1 = x[..., :h]
    x2 = x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_interleaved(x, cos, sin):
    """Complex-formulation RoPE: pair (2i, 2i+1) read as x_2i + i x_2i+1 and
    multiplied by exp(i angle_i); the output keeps the interleaved layout."""
    h = x.shape[-1] // 2
    shp = (cos.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = cos.reshape(shp)
    s = sin.reshape(shp)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x, dtype=np.float64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xo * c + xe * s
    return out


def apply_rope(x, positions, cfg: Cfg):
    """RoPE of ``cfg``'s convention and frequencies at ``positions``.

    x: [T, ..., d_r] float64; positions: [T]."""
    cos, sin = rope_cos_sin(positions, cfg_inv_freq(cfg), cfg_cos_sin_scale(cfg))
    if cfg.rope_convention == HALF_SPLIT:
        return rope_half_split(x, cos, sin)
    if cfg.rope_convention == INTERLEAVED:
        return rope_interleaved(x, cos, sin)
    raise ValueError(cfg.rope_convention)


def deinterleave_perm(d: int) -> np.ndarray:
    """P with (P x)_i = x_2i and (P x)_{i+d/2} = x_{2i+1}: x[..., P] gives P x."""
    return np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])


# ------------------------------------------------------------- RMSNorm ----

def rmsnorm(x, g, eps):
    """x * (mean(x^2) + eps)^-1/2 * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def latent(cfg: Cfg, w: dict, x):
    """c_kv = x W_dkv^T, the cached latent.  The pages put no norm on it; a
    checkpoint may carry RMSNorm gains for it (w["kv_norm"]), which are then
    applied like the norm on c_q."""
    c_kv = x @ _f64(w["w_down_kv"]).T
    if w.get("kv_norm") is not None:
        c_kv = rmsnorm(c_kv, _f64(w["kv_norm"]), cfg.rms_norm_eps)
    return c_kv


def softmax_scale(cfg: Cfg) -> float:
    """1/sqrt(d_nope + d_rope), times mscale(factor, mscale_all_dim)^2 with
    YaRN (the MLA listing divides the scores by sqrt(dk))."""
    if cfg.softmax_scale_override is not None:
        return float(cfg.softmax_scale_override)
    s = 1.0 / math.sqrt(cfg.qk_nope_head_dim + cfg.qk_rope_head_dim)
    if cfg.rope_factor > 1.0:
        m = yarn_mscale(cfg.rope_factor, cfg.mscale_all_dim)
        s = s * m * m
    return s


# ------------------------------------------------------------ attention ---

def causal_attention(q, k, v, scale, q_pos=None):
    """Softmax attention of one head with the causal tril mask.

    q: [Sq, dk], k: [Sk, dk], v: [Sk, dv]; query row r sits at position
    q_pos[r] (default r) and sees keys j <= q_pos[r]."""
    sq = q.shape[0]
    sk = k.shape[0]
    if q_pos is None:
        q_pos = np.arange(sq)
    s = scale * (q @ k.T)
    mask = np.arange(sk)[None, :] > np.asarray(q_pos)[:, None]
    s = np.where(mask, -np.inf, s)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v


# --------------------------------------------------------------- prefill ---

def _f64(a):
    return np.asarray(a, dtype=np.float64)


def mla_prefill(cfg: Cfg, w: dict, x, want_intermediates: bool = False):
    """Full MLA prefill forward of x [B, S, D] at positions 0..S-1.

    Returns y [B, S, D] (and a dict of intermediates if asked)."""
    x = _f64(x)
    B, S, D = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    pos = np.arange(S)

    # query path: c_q = w_down_q x, RMSNorm, then w_up_q / w_qr
    c_q = x @ _f64(w["w_down_q"]).T
    c_qn = rmsnorm(c_q, _f64(w["q_norm"]), cfg.rms_norm_eps)
    q_nope = (c_qn @ _f64(w["w_up_q"]).T).reshape(B, S, H, dn)
    q_pe = (c_qn @ _f64(w["w_qr"]).T).reshape(B, S, H, dr)
    # KV path: the cached latent, and the shared RoPE key bypassing it
    c_kv = latent(cfg, w, x)
    k_pe = x @ _f64(w["w_kr"]).T  # [B, S, dr]
    q_pe = np.stack([apply_rope(q_pe[b], pos, cfg) for b in range(B)])
    k_pe = np.stack([apply_rope(k_pe[b], pos, cfg) for b in range(B)])
    k_nope = (c_kv @ _f64(w["w_up_k"]).T).reshape(B, S, H, dn)
    v = (c_kv @ _f64(w["w_up_v"]).T).reshape(B, S, H, dv)

    scale = softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            q = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            k = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = causal_attention(q, k, v[b, :, h], scale)
    o = o.reshape(B, S, H * dv)
    y = o @ _f64(w["wo"]).T
    if not want_intermediates:
        return y
    return y, dict(c_q=c_q, c_qn=c_qn, q_nope=q_nope, q_pe=q_pe, c_kv=c_kv,
                   k_pe=k_pe, k_nope=k_nope, v=v, o=o)


def mla_prefill_varlen(cfg: Cfg, w: dict, x, cu_seqlens):
    """Prefill of sequences of different lengths packed end to end: x [T, D],
    sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1]-1.  Each sequence is a
    prefill of its own (positions from 0, causal mask within the sequence:
    the MLA section's forward applied per sequence).

    Returns y [T, D] and the latent rows [T, r_kv + d_r] (c_kv, then the
    post-RoPE k_pe)."""
    x = _f64(x)
    cu = [int(v) for v in cu_seqlens]
    T, D = x.shape
    width = cfg.kv_lora_rank + cfg.qk_rope_head_dim
    y = np.empty((T, D))
    lat = np.empty((T, width))
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        if e == a:
            continue
        yb, inter = mla_prefill(cfg, w, x[None, a:e], want_intermediates=True)
        y[a:e] = yb[0]
        lat[a:e] = np.concatenate([inter["c_kv"][0], inter["k_pe"][0]], axis=-1)
    return y, lat


def mla_prefill_rows(cfg: Cfg, w: dict, x, rows, batch: int = 0):
    """y[batch, r] for the query rows ``rows`` of a prefill of x [B, S, D].

    Same arithmetic as :func:`mla_prefill`, but the queries are only formed
    for ``rows`` and K/V are expanded one head at a time, so long sequences
    fit in memory.  Returns (y_rows [R, D], latent [S, r_kv + d_r])."""
    xb = _f64(x[batch])
    S, D = xb.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    rows = np.asarray(rows, dtype=np.int64)
    pos = np.arange(S)
    c_kv = latent(cfg, w, xb)
    k_pe = apply_rope(xb @ _f64(w["w_kr"]).T, pos, cfg)
    xr = xb[rows]
    c_qn = rmsnorm(xr @ _f64(w["w_down_q"]).T, _f64(w["q_norm"]), cfg.rms_norm_eps)
    q_nope = (c_qn @ _f64(w["w_up_q"]).T).reshape(len(rows), H, dn)
    q_pe = apply_rope((c_qn @ _f64(w["w_qr"]).T).reshape(len(rows), H, dr),
                      rows, cfg)
    scale = softmax_scale(cfg)
    wuk = _f64(w["w_up_k"])
    wuv = _f64(w["w_up_v"])
    o = np.empty((len(rows), H, dv))
    kmax = int(rows.max()) + 1
    for h in range(H):
        k_nope = c_kv[:kmax] @ wuk[h * dn:(h + 1) * dn].T
        v = c_kv[:kmax] @ wuv[h * dv:(h + 1) * dv].T
        k = np.concatenate([k_nope, k_pe[:kmax]], axis=-1)
        q = np.concatenate([q_nope[:, h], q_pe[:, h]], axis=-1)
        o[:, h] = causal_attention(q, k, v, scale, q_pos=rows)
    y = o.reshape(len(rows), H * dv) @ _f64(w["wo"]).T
    return y, np.concatenate([c_kv, k_pe], axis=-1)


# ---------------------------------------------------------------- decode ---

def _decode_new_token(cfg: Cfg, w: dict, xb, p):
    """q_nope [H, dn], post-RoPE q_pe [H, dr] and the new cache row
    [c_kv ‖ post-RoPE k_pe] of one token at position p."""
    H = cfg.num_attention_heads
    dn, dr = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim
    c_qn = rmsnorm(xb @ _f64(w["w_down_q"]).T, _f64(w["q_norm"]), cfg.rms_norm_eps)
    q_nope = (c_qn @ _f64(w["w_up_q"]).T).reshape(H, dn)
    q_pe = apply_rope((c_qn @ _f64(w["w_qr"]).T).reshape(1, H, dr), [p], cfg)[0]
    c_kv = latent(cfg, w, xb)
    k_pe = apply_rope((xb @ _f64(w["w_kr"]).T)[None, :], [p], cfg)[0]
    return q_nope, q_pe, np.concatenate([c_kv, k_pe])


def mla_decode_expanded(cfg: Cfg, w: dict, x, cache, lens):
    """One decode step by the definition: per head, expand every cached latent
    row to K_nope = W_uk_h c_kv and V = W_uv_h c_kv, attend over rows
    0..L_b (the new token included), project with wo.

    x: [B, D]; cache: [B, cap, r_kv + d_r] (rows < lens[b] valid).
    Returns (y [B, D], new_rows [B, r_kv + d_r])."""
    x = _f64(x)
    B = x.shape[0]
    H = cfg.num_attention_heads
    dn, dv = cfg.qk_nope_head_dim, cfg.v_head_dim
    r = cfg.kv_lora_rank
    wuk = _f64(w["w_up_k"]).reshape(H, dn, r)
    wuv = _f64(w["w_up_v"]).reshape(H, dv, r)
    scale = softmax_scale(cfg)
    y = np.empty((B, cfg.hidden_size))
    new_rows = np.empty((B, cache.shape[-1]))
    for b in range(B):
        L = int(lens[b])
        q_nope, q_pe, row = _decode_new_token(cfg, w, x[b], L)
        new_rows[b] = row
        rows = np.concatenate([_f64(cache[b, :L]), row[None]], axis=0)
        c, kp = rows[:, :r], rows[:, r:]
        o = np.empty((H, dv))
        for h in range(H):
            k = np.concatenate([c @ wuk[h].T, kp], axis=-1)
            v = c @ wuv[h].T
            q = np.concatenate([q_nope[h], q_pe[h]])[None]
            o[h] = causal_attention(q, k, v, scale, q_pos=[L])[0]
        y[b] = o.reshape(-1) @ _f64(w["wo"]).T
    return y, new_rows


def mla_decode_absorbed(cfg: Cfg, w: dict, x, cache, lens,
                        want_intermediates: bool = False):
    """One decode step in absorbed form: q_lat_h = W_uk_h^T q_nope_h, scores
    scale (q_lat_h . c_kv_t + q_pe_h . k_pe_t) over t = 0..L_b, o_lat_h =
    sum_t p_t c_kv_t, o_h = W_uv_h o_lat_h, y = wo o.  Equal to
    :func:`mla_decode_expanded` in exact arithmetic (associativity)."""
    x = _f64(x)
    B = x.shape[0]
    H = cfg.num_attention_heads
    dn, dv = cfg.qk_nope_head_dim, cfg.v_head_dim
    r = cfg.kv_lora_rank
    wuk = _f64(w["w_up_k"]).reshape(H, dn, r)
    wuv = _f64(w["w_up_v"]).reshape(H, dv, r)
    wo = _f64(w["wo"])
    scale = softmax_scale(cfg)
    y = np.empty((B, cfg.hidden_size))
    new_rows = np.empty((B, cache.shape[-1]))
    q_lats = np.empty((B, H, r))
    o_lats = np.empty((B, H, r))
    for b in range(B):
        L = int(lens[b])
        q_nope, q_pe, row = _decode_new_token(cfg, w, x[b], L)
        new_rows[b] = row
        rows = np.concatenate([_f64(cache[b, :L]), row[None]], axis=0)
        c, kp = rows[:, :r], rows[:, r:]
        q_lat = np.einsum("hd,hdr->hr", q_nope, wuk)
        s = scale * (q_lat @ c.T + q_pe @ kp.T)  # [H, L+1]
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        o_lat = p @ c  # [H, r]
        o = np.einsum("hvr,hr->hv", wuv, o_lat)
        y[b] = o.reshape(-1) @ wo.T
        q_lats[b] = q_lat
        o_lats[b] = o_lat
    if want_intermediates:
        return y, new_rows, dict(q_lat=q_lats, o_lat=o_lats)
    return y, new_rows


def mla_decode_absorbed_multi(cfg: Cfg, w: dict, x, cache, lens):
    """Several new tokens per sequence in one absorbed decode step (the
    multi-token / speculative-verification use of the cache formula).

    Token t of sequence b sits at position L_b + t; its latent row is written
    at cache row L_b + t, and it attends to rows 0..L_b + t -- the cached
    prefix and the new tokens up to itself, which is the causal tril mask of
    the MLA listing ("The Evolving Transformer -- DeepSeek V2 & V3", section
    01) applied to the new tokens.  Per token the arithmetic is the absorbed
    form of :func:`mla_decode_absorbed`.

    x: [B, T, D]; cache: [B, cap, r_kv + d_r] (rows < lens[b] valid).
    Returns (y [B, T, D], new_rows [B, T, r_kv + d_r])."""
    x = _f64(x)
    B, T = x.shape[0], x.shape[1]
    H = cfg.num_attention_heads
    dn, dv = cfg.qk_nope_head_dim, cfg.v_head_dim
    r = cfg.kv_lora_rank
    wuk = _f64(w["w_up_k"]).reshape(H, dn, r)
    wuv = _f64(w["w_up_v"]).reshape(H, dv, r)
    wo = _f64(w["wo"])
    scale = softmax_scale(cfg)
    y = np.empty((B, T, cfg.hidden_size))
    new_rows = np.empty((B, T, cache.shape[-1]))
    for b in range(B):
        L = int(lens[b])
        toks = [_decode_new_token(cfg, w, x[b, t], L + t) for t in range(T)]
        for t in range(T):
            new_rows[b, t] = toks[t][2]
        rows_all = np.concatenate([_f64(cache[b, :L]), new_rows[b]], axis=0)  # [L+T, W]
        for t in range(T):
            q_nope, q_pe, _ = toks[t]
            rows = rows_all[:L + t + 1]
            c, kp = rows[:, :r], rows[:, r:]
            q_lat = np.einsum("hd,hdr->hr", q_nope, wuk)
            s = scale * (q_lat @ c.T + q_pe @ kp.T)  # [H, L+t+1]
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            o = np.einsum("hvr,hr->hv", wuv, p @ c)
            y[b, t] = o.reshape(-1) @ wo.T
    return y, new_rows

