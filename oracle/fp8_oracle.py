"""Plain float64 oracle of block-scaled FP8 (E4M3) projection products.

TEST INFRASTRUCTURE ONLY -- never on the product path.  Slow and obvious on
purpose: the format is decoded from its bit fields, the encoder rounds by the
definition, and the product is one float64 matrix multiply of the decoded,
scaled operands.

Source: the "Deep Seek V3" notes (knlb.dev), section "infrastructure", the
FP8 bullets: quantisation is fine grained (tile-wise for activations,
block-wise for weights), the scales come online from the maxima of each tile
or block, every tensor uses E4M3, the products accumulate at a precision above
FP8, and attention, normalisation, embedding and output head stay in higher
precision.

Readings where the notes are silent (each is listed in the design notes):

* E4M3 is the OCP 8-bit E4M3 format: sign, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals at exponent field 0, no infinities, NaN only for
  the all-ones exponent and mantissa, largest finite value 448.
* Encoding rounds to the nearest representable value, ties to the even
  mantissa.  The scaled inputs never exceed 448, so no saturation rule is
  needed (the encoder rejects larger magnitudes).
* Activation tiles are 1 x 128 along the reduction axis (one scale per row per
  128 columns); weight blocks are 128 x 128 (one scale per 128 output rows per
  128 reduction columns; a partial last row block keeps its own scale).
* A scale is a power of two 2^e: the smallest one with amax <= 448 * 2^e,
  e = 0 for an all-zero tile, e clamped to [-127, 127].  Dividing by it is
  exact, and it is what the matrix cores apply as a block exponent.
* The product is C[m, n] = sum_k dec(qa[m, k]) 2^ea[m, k // 128]
  * dec(qb[n, k]) 2^eb[n // 128, k // 128], the reduction length a multiple
  of 128.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
TILE = 128


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte from its fields (float64; NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = (m / 8.0) * np.ldexp(1.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 byte of each value (ties to even mantissa); |x| <= 448."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values of magnitude <= 448")
    a = np.abs(x)
    # spacing of the grid around a: 2^(E-3) in the binade [2^E, 2^(E+1)),
    # 2^-9 below the smallest normal 2^-6
    _, ex = np.frexp(a)                      # a = f 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, E - 3)
    n = np.rint(a / q)                       # round half to even on the grid
    v = n * q                                # rounded magnitude (exact)
    # fields of the rounded magnitude (a carry into the next binade is
    # handled by re-reading its exponent)
    _, ev = np.frexp(v)
    Ev = ev - 1
    is_sub = (v < 2.0 ** -6)
    mant_sub = np.rint(v / 2.0 ** -9)
    mant_norm = np.rint(v / np.ldexp(1.0, Ev) * 8.0) - 8.0
    efield = np.where(is_sub, 0, Ev + 7)
    mfield = np.where(is_sub, mant_sub, mant_norm)
    code = (efield.astype(np.int64) << 3) | mfield.astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e (e = 0 where amax == 0), in [-127, 127]."""
    a = np.asarray(amax, dtype=np.float64)
    f, ex = np.frexp(a)                      # a = f 2^ex; 448 = 0.875 * 2^9
    e = ex - 9 + (f > 0.875)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_act_tiles(x):
    """1 x 128 tiles along the last axis of x [M, K] -> (codes [M, K] uint8,
    exponents [M, K/128] int64)."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % TILE:
        raise ValueError("the reduction length must be a multiple of 128")
    t = x.reshape(M, K // TILE, TILE)
    e = block_exponent(np.abs(t).max(axis=2))
    codes = e4m3_encode(t * np.ldexp(1.0, -e)[:, :, None])
    return codes.reshape(M, K), e


def quantize_weight_blocks(w):
    """128 x 128 blocks of w [N, K] -> (codes [N, K] uint8,
    exponents [ceil(N/128), K/128] int64)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if K % TILE:
        raise ValueError("the reduction length must be a multiple of 128")
    nb = (N + TILE - 1) // TILE
    e = np.zeros((nb, K // TILE), dtype=np.int64)
    codes = np.zeros((N, K), dtype=np.uint8)
    for i in range(nb):
        rows = w[i * TILE:(i + 1) * TILE]
        blk = rows.reshape(rows.shape[0], K // TILE, TILE)
        e[i] = block_exponent(np.abs(blk).max(axis=(0, 2)))
        codes[i * TILE:(i + 1) * TILE] = e4m3_encode(
            blk * np.ldexp(1.0, -e[i])[None, :, None]).reshape(rows.shape[0], K)
    return codes, e


def dequant_act(codes, e):
    """Float64 values of 1 x 128 tiles: dec(code) * 2^e of the tile."""
    v = e4m3_decode(codes)
    return v * np.repeat(np.ldexp(1.0, e), TILE, axis=1)


def dequant_weight(codes, e):
    """Float64 values of 128 x 128 blocks: dec(code) * 2^e of the block."""
    v = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.ldexp(1.0, e), TILE, axis=0), TILE, axis=1)
    return v * s[:v.shape[0]]


def fp8_gemm(qa, ea, qb, eb):
    """C [M, N] = dequant_act(qa, ea) @ dequant_weight(qb, eb)^T in float64."""
    return dequant_act(qa, ea) @ dequant_weight(qb, eb).T


def quantized_product(x, w):
    """x [M, K] times w [N, K]^T with x quantised in 1 x 128 tiles and w in
    128 x 128 blocks, the product in float64 (the block-scaled FP8 product of
    the notes' scheme, applied to one projection)."""
    qa, ea = quantize_act_tiles(x)
    qb, eb = quantize_weight_blocks(w)
    return fp8_gemm(qa, ea, qb, eb)


def qdq_act(x):
    """x [M, K] after 1 x 128 tile quantisation (dequantised, float64)."""
    return dequant_act(*quantize_act_tiles(x))


def qdq_weight(w):
    """w [N, K] after 128 x 128 block quantisation (dequantised, float64)."""
    return dequant_weight(*quantize_weight_blocks(w))


def mla_prefill_fp8(cfg, w, x):
    """The MLA prefill with its four projection products in block-scaled FP8.

    The notes' scheme keeps attention, normalisation and the rest in higher
    precision and runs the linear layers in FP8 with fine-grained scales.
    So, following the MLA listing of "The Evolving Transformer -- DeepSeek V2
    & V3" (section 01) step by step as the float64 oracle does, each
    projection's input activation is quantised in 1 x 128 tiles and each
    weight matrix in 128 x 128 blocks (every matrix on its own), and the
    product is taken of the dequantised values:

      down  [c_q ‖ c_kv ‖ k_pe] = q(x) [q(W_dq); q(W_dkv); q(W_kr)]^T
      q up  [q_nope ‖ q_pe]     = q(RMSNorm(c_q)) [q(W_uq); q(W_qr)]^T
      kv up [k_nope ‖ v]        = q(c_kv) [q(W_uk); q(W_uv)]^T
      out   y                   = q(o) q(W_o)^T

    RMSNorm, RoPE and the causal softmax attention are the float64 oracle's.
    x: [B, S, D]; returns y [B, S, D]."""
    from . import mla_oracle as mo
    x = np.asarray(x, dtype=np.float64)
    B, S, D = x.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items() if v is not None}
    xf = x.reshape(B * S, D)
    c_q = quantized_product(xf, f["w_down_q"])
    c_kv = quantized_product(xf, f["w_down_kv"])
    k_pe = quantized_product(xf, f["w_kr"])
    c_qn = mo.rmsnorm(c_q, f["q_norm"], cfg.rms_norm_eps)
    if "kv_norm" in f:
        c_kv = mo.rmsnorm(c_kv, f["kv_norm"], cfg.rms_norm_eps)
    q_nope = quantized_product(c_qn, f["w_up_q"]).reshape(B, S, H, dn)
    q_pe = quantized_product(c_qn, f["w_qr"]).reshape(B, S, H, dr)
    k_nope = quantized_product(c_kv, f["w_up_k"]).reshape(B, S, H, dn)
    v = quantized_product(c_kv, f["w_up_v"]).reshape(B, S, H, dv)
    pos = np.arange(S)
    q_pe = np.stack([mo.apply_rope(q_pe[b], pos, cfg) for b in range(B)])
    k_pe = np.stack([mo.apply_rope(k_pe.reshape(B, S, dr)[b], pos, cfg) for b in range(B)])
    scale = mo.softmax_scale(cfg)
    o = np.empty((B, S, H, dv))
    for b in range(B):
        for h in range(H):
            q = np.concatenate([q_nope[b, :, h], q_pe[b, :, h]], axis=-1)
            k = np.concatenate([k_nope[b, :, h], k_pe[b]], axis=-1)
            o[b, :, h] = mo.causal_attention(q, k, v[b, :, h], scale)
    y = quantized_product(o.reshape(B * S, H * dv), f["wo"])
    return y.reshape(B, S, D)


def mla_prefill_fp8_rows(cfg, w, x, rows, batch: int = 0):
    """y[batch, r] of :func:`mla_prefill_fp8` for the query rows ``rows``,
    with the latent [S, r_kv + d_r] of every token.  Same quantisation and
    arithmetic; the queries are formed only for ``rows`` (their activation
    tiles are row-local, so quantising a subset of rows changes nothing) and
    the keys and values head by head, so V3 sizes fit in memory."""
    from . import mla_oracle as mo
    xb = np.asarray(x[batch], dtype=np.float64)
    S, D = xb.shape
    H = cfg.num_attention_heads
    dn, dr, dv = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim
    rows = np.asarray(rows, dtype=np.int64)
    f = {k: np.asarray(v, dtype=np.float64) for k, v in w.items() if v is not None}
    pos = np.arange(S)
    xq = qdq_act(xb)  # x quantised once; its tiles are row-local
    c_kv = xq @ qdq_weight(f["w_down_kv"]).T
    if "kv_norm" in f:
        c_kv = mo.rmsnorm(c_kv, f["kv_norm"], cfg.rms_norm_eps)
    k_pe = mo.apply_rope(xq @ qdq_weight(f["w_kr"]).T, pos, cfg)
    c_qn = mo.rmsnorm(xq[rows] @ qdq_weight(f["w_down_q"]).T, f["q_norm"], cfg.rms_norm_eps)
    q_nope = quantized_product(c_qn, f["w_up_q"]).reshape(len(rows), H, dn)
    q_pe = mo.apply_rope(quantized_product(c_qn, f["w_qr"]).reshape(len(rows), H, dr), rows, cfg)
    kmax = int(rows.max()) + 1
    # the kv up-projection of the quantised latent: operands quantised once
    ca = qdq_act(c_kv[:kmax])
    wuk = qdq_weight(f["w_up_k"])
    wuv = qdq_weight(f["w_up_v"])
    scale = mo.softmax_scale(cfg)
    o = np.empty((len(rows), H, dv))
    for h in range(H):
        k = np.concatenate([ca @ wuk[h * dn:(h + 1) * dn].T, k_pe[:kmax]], axis=-1)
        v = ca @ wuv[h * dv:(h + 1) * dv].T
        q = np.concatenate([q_nope[:, h], q_pe[:, h]], axis=-1)
        o[:, h] = mo.causal_attention(q, k, v, scale, q_pos=rows)
    y = quantized_product(o.reshape(len(rows), H * dv), f["wo"])
    return y, np.concatenate([c_kv, k_pe], axis=-1)
