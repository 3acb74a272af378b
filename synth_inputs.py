"""Seeded synthetic inputs for the MLA forward: shapes, seeds and draws only.

This module holds none of the method's arithmetic.  Both the tests/bench (for
the HIP library) and the float64 oracle take their inputs from here, so the
two sides see exactly the same values.

Recipe (the pages publish no dataset for this path, so seeded draws stand in):

* NumPy ``default_rng(seed)`` (PCG64), draws in a fixed order:
  x, w_down_q, w_up_q, w_qr, w_down_kv, w_kr, w_up_k, w_up_v, wo, then the
  decode cache lengths and the cache itself.
* x ~ N(0, 1); every weight ~ N(0, w_std^2); RMSNorm gains are 1 unless a
  test asks for random gains (1 + 0.1 N(0,1), drawn after wo).
* Values are rounded once to bf16 (round to nearest even) for bf16 configs;
  the device gets those bf16 values and the oracle gets the same values
  upcast to float64.
* Shapes follow the DeepSeek-V3 dimension table of the "DeepSeek-V3 Decoupled
  Implementation" README (hidden 7168, 128 heads, q_lora_rank 1536,
  kv_lora_rank 512, nope 128, rope 64, v 128) and smaller stand-ins.
"""

from __future__ import annotations

import numpy as np

V3 = dict(hidden_size=7168, num_attention_heads=128, q_lora_rank=1536,
          kv_lora_rank=512, qk_nope_head_dim=128, qk_rope_head_dim=64,
          v_head_dim=128)

CONFIGS = {
    # tiny fp32 correctness case
    "tiny": dict(batch=1, seq=16, hidden_size=64, num_attention_heads=4,
                 q_lora_rank=32, kv_lora_rank=16, qk_nope_head_dim=16,
                 qk_rope_head_dim=8, v_head_dim=16, dtype="fp32",
                 rope="half_split", w_std=0.02, seed=1000),
    # small bf16 correctness case, both conventions
    "small": dict(batch=2, seq=512, hidden_size=1024, num_attention_heads=16,
                  q_lora_rank=256, kv_lora_rank=128, qk_nope_head_dim=64,
                  qk_rope_head_dim=32, v_head_dim=64, dtype="bf16",
                  rope="half_split", w_std=0.02, seed=2000),
    # DeepSeek-V3-shaped prefill
    "v3_prefill": dict(batch=1, seq=4096, **V3, dtype="bf16",
                       rope="interleaved", w_std=0.006, seed=3000),
    # DeepSeek-V3-shaped absorbed decode over a latent cache
    "v3_decode": dict(batch=64, seq=1, **V3, dtype="bf16",
                      rope="interleaved", w_std=0.006, seed=4000,
                      len_lo=1024, len_hi=8192, capacity=8193),
    # long-context prefill with YaRN frequencies
    "v3_yarn": dict(batch=1, seq=32768, **V3, dtype="bf16",
                    rope="interleaved", w_std=0.006, seed=5000,
                    rope_factor=40.0, original_max_position_embeddings=4096,
                    beta_fast=32.0, beta_slow=1.0, mscale=1.0,
                    mscale_all_dim=1.0, sample_rows=256, sample_seed=5001),
}


def round_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); the result is
    float32 holding bf16-representable values.  Finite inputs only (the
    uint32 sum cannot overflow below the NaN bit patterns)."""
    a = np.array(a, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _store(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def weight_shapes(c) -> dict:
    """nn.Linear weight shapes [out, in] of one MLA layer."""
    D, H = c["hidden_size"], c["num_attention_heads"]
    rq, rkv = c["q_lora_rank"], c["kv_lora_rank"]
    dn, dr, dv = c["qk_nope_head_dim"], c["qk_rope_head_dim"], c["v_head_dim"]
    return dict(w_down_q=(rq, D), w_up_q=(H * dn, rq), w_qr=(H * dr, rq),
                w_down_kv=(rkv, D), w_kr=(dr, D), w_up_k=(H * dn, rkv),
                w_up_v=(H * dv, rkv), wo=(D, H * dv))


WEIGHT_ORDER = ("w_down_q", "w_up_q", "w_qr", "w_down_kv", "w_kr", "w_up_k",
                "w_up_v", "wo")


def make_inputs(c: dict, *, seq=None, batch=None, gains="ones",
                weight_scale=None, dtype=None, seed=None):
    """Draw x and the weights of config ``c`` (optionally overriding sizes).

    Returns (x [B, S, D] float32, weights dict of float32 arrays), values
    already rounded to the config's storage dtype."""
    dtype = dtype or c["dtype"]
    B = batch if batch is not None else c["batch"]
    S = seq if seq is not None else c["seq"]
    rng = np.random.default_rng(c["seed"] if seed is None else seed)
    D = c["hidden_size"]
    x = _store(rng.standard_normal((B, S, D), dtype=np.float32), dtype)
    w = {}
    std = np.float32(c["w_std"])
    for name in WEIGHT_ORDER:
        shp = weight_shapes(c)[name]
        a = rng.standard_normal(shp, dtype=np.float32) * std
        if weight_scale and name in weight_scale:
            a = a * np.float32(weight_scale[name])
        w[name] = _store(a, dtype)
    if gains == "random":
        g = 1.0 + 0.1 * rng.standard_normal(c["q_lora_rank"], dtype=np.float32)
    else:
        g = np.ones(c["q_lora_rank"], dtype=np.float32)
    w["q_norm"] = _store(g, dtype)
    return x, w


def make_decode_inputs(c: dict, *, batch=None, capacity=None, len_lo=None,
                       len_hi=None, dtype=None, seed=None, gains="ones"):
    """x_new [B, D], weights, cache lengths [B] int32 and the latent cache
    [B, capacity, r_kv + d_r] with rows ~N(0,1) (rows >= len are also drawn
    but are never read as history)."""
    dtype = dtype or c["dtype"]
    B = batch if batch is not None else c["batch"]
    cap = capacity if capacity is not None else c["capacity"]
    lo = len_lo if len_lo is not None else c["len_lo"]
    hi = len_hi if len_hi is not None else c["len_hi"]
    x, w = make_inputs(c, seq=1, batch=B, dtype=dtype, seed=seed, gains=gains)
    rng = np.random.default_rng((c["seed"] if seed is None else seed) + 1)
    lens = rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)
    width = c["kv_lora_rank"] + c["qk_rope_head_dim"]
    cache = _store(rng.standard_normal((B, cap, width), dtype=np.float32), dtype)
    return x[:, 0, :], w, lens, cache


def sample_rows(c: dict, seq: int):
    """Seeded query rows to check at long sequence lengths, plus the tile and
    YaRN boundary rows {0, 4095, 4096, seq-1}."""
    rng = np.random.default_rng(c.get("sample_seed", c["seed"] + 1))
    n = min(c.get("sample_rows", 256), seq)
    rows = set(rng.choice(seq, size=n, replace=False).tolist())
    rows |= {r for r in (0, 4095, 4096, seq - 1) if r < seq}
    return np.array(sorted(rows), dtype=np.int64)


def make_fp8_operands(M: int, N: int, K: int, seed: int, *, spread: bool = True,
                      w_std: float = 0.006):
    """Operands of one block-scaled FP8 projection product, as bf16 values.

    x [M, K] ~ N(0, 1) (an activation such as the attention output feeding the
    output projection) and w [N, K] ~ N(0, w_std^2) (nn.Linear weight).  With
    spread, every 1 x 128 tile of x is multiplied by 2^u, u ~ U{-6..6}, and
    every 128 x 128 block of w by 2^v, v ~ U{-4..4}, so that tiles and blocks
    carry different scales.  Drawn in the order x, w, tile exponents, block
    exponents; rounded once to bf16 (returned as float32)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std))
    if spread:
        u = rng.integers(-6, 7, (M, K // 128))
        v = rng.integers(-4, 5, ((N + 127) // 128, K // 128))
        x = x * np.repeat(np.ldexp(np.float32(1), u), 128, axis=1).astype(np.float32)
        wv = np.repeat(np.repeat(np.ldexp(np.float32(1), v), 128, axis=0), 128, axis=1)[:N]
        w = w * wv.astype(np.float32)
    return round_bf16(x), round_bf16(w)


def make_attention_backward_inputs(BH: int, S: int, dqk: int, dv: int, seed: int, bf16: bool = False):
    """q, k [BH, S, dqk], v [BH, S, dv] and the upstream gradient dout
    [BH, S, dv], all N(0, 1), drawn in that order (float32; rounded once to
    bf16 when asked)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((BH, S, dqk), dtype=np.float32)
    k = rng.standard_normal((BH, S, dqk), dtype=np.float32)
    v = rng.standard_normal((BH, S, dv), dtype=np.float32)
    do = rng.standard_normal((BH, S, dv), dtype=np.float32)
    out = (q, k, v, do)
    return tuple(round_bf16(a) for a in out) if bf16 else out
