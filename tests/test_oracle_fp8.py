"""Pins of the FP8 (E4M3) oracle against the format's definition, brute force
and an independent library cast (no GPU)."""

import numpy as np
import pytest
import torch

from oracle import fp8_oracle as f8

RNG = np.random.default_rng(8)
ALL = np.arange(256, dtype=np.uint8)


def test_decode_fixed_points():
    # values the E4M3 bit layout fixes (bias 7, 3 mantissa bits, no infinities)
    d = f8.e4m3_decode(ALL)
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9     # subnormals
    assert d[0x08] == 2.0 ** -6                                  # smallest normal
    assert d[0x38] == 1.0 and d[0x3C] == 1.5 and d[0x40] == 2.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0                # largest finite
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                               # monotone in the code
    np.testing.assert_array_equal(d[0x80:0xFF], -d[:0x7F])


def test_decode_matches_torch_float8():
    # an independent implementation of the same format
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).double().numpy()
    d = f8.e4m3_decode(ALL)
    fin = ~np.isnan(d)
    np.testing.assert_array_equal(d[fin], t[fin])
    assert np.all(np.isnan(t[~fin]))


def _brute_encode(v):
    # nearest finite positive code by exhaustive search, ties to the even code
    table = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = abs(v)
    dist = np.abs(table - a)
    best = np.flatnonzero(dist == dist.min())
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return int(c) | (0x80 if np.signbit(v) else 0)


def test_encode_brute_force():
    table = f8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (table[1:] + table[:-1]) / 2
    vals = np.concatenate([
        table, -table, mids, -mids, mids * (1 + 1e-12), mids * (1 - 1e-12),
        RNG.uniform(-448, 448, 400),
        np.ldexp(RNG.uniform(0.5, 1, 400), RNG.integers(-12, 9, 400)) * RNG.choice([-1, 1], 400),
    ])
    vals = vals[np.abs(vals) <= 448]
    got = f8.e4m3_encode(vals)
    exp = np.array([_brute_encode(v) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, exp)


def test_encode_matches_torch_cast():
    # the library's round-to-nearest-even cast (fp64 -> e4m3fn) on the same values
    vals = np.concatenate([RNG.uniform(-448, 448, 2000),
                           np.ldexp(RNG.standard_normal(2000), RNG.integers(-14, 6, 2000))])
    vals = vals[np.abs(vals) <= 448]
    t = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(f8.e4m3_encode(vals), t)


def test_encode_roundtrip_and_range():
    fin = ALL[~np.isnan(f8.e4m3_decode(ALL))]
    np.testing.assert_array_equal(f8.e4m3_encode(f8.e4m3_decode(fin)), fin)
    with pytest.raises(ValueError):
        f8.e4m3_encode(np.array([448.5]))


def test_block_exponent_definition():
    a = np.concatenate([np.ldexp(RNG.uniform(0.5, 1, 500), RNG.integers(-40, 40, 500)),
                        448.0 * np.ldexp(1.0, np.arange(-20, 20)),
                        448.0 * np.ldexp(1.0, np.arange(-20, 20)) * (1 + 2.0 ** -40),
                        [1.0, 448.0, 449.0, 224.0]])
    e = f8.block_exponent(a)
    assert np.all(a <= 448.0 * np.ldexp(1.0, e))               # fits
    assert np.all(a > 448.0 * np.ldexp(1.0, e - 1))            # and is the smallest
    assert f8.block_exponent(np.array([0.0]))[0] == 0
    assert f8.block_exponent(np.array([448.0]))[0] == 0
    assert f8.block_exponent(np.array([449.0]))[0] == 1
    assert f8.block_exponent(np.array([1e-300]))[0] == -127   # clamped


def test_quantize_act_error_bound():
    x = RNG.standard_normal((37, 512)) * np.ldexp(1.0, RNG.integers(-8, 8, (37, 1)))
    q, e = f8.quantize_act_tiles(x)
    assert e.shape == (37, 4)
    s = x / np.repeat(np.ldexp(1.0, e), 128, axis=1)
    d = f8.e4m3_decode(q)
    # half a grid step: 2^-4 relative for normals, 2^-10 absolute below 2^-6
    bound = np.maximum(np.abs(s) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(s - d) <= bound)
    amax = np.abs(s).reshape(37, 4, 128).max(axis=2)
    assert np.all((amax > 224) & (amax <= 448))
    scale = np.repeat(np.ldexp(1.0, e), 128, axis=1)
    assert np.all(np.abs(f8.dequant_act(q, e) - x) <= bound * scale)


def _exact_operand(rows, K, e, block_rows):
    # codes whose tiles (blocks) quantise back to themselves under exponent e
    codes = RNG.integers(0, 0x7F, (rows, K)).astype(np.uint8) | (RNG.integers(0, 2, (rows, K)) << 7).astype(np.uint8)
    codes[0::block_rows, 0::128] = 0x7E      # each tile/block holds a 448
    return codes, e


def test_quantize_roundtrip_exact_inputs():
    M, N, K = 70, 150, 384
    qa, ea = _exact_operand(M, K, RNG.integers(-20, 5, (M, K // 128)), 1)
    qa[:, 0::128] = 0x7E
    xa = f8.dequant_act(qa, ea)
    qa2, ea2 = f8.quantize_act_tiles(xa)
    np.testing.assert_array_equal(ea2, ea)
    np.testing.assert_array_equal(f8.e4m3_decode(qa2), f8.e4m3_decode(qa))
    eb = RNG.integers(-20, 5, ((N + 127) // 128, K // 128))
    qb, _ = _exact_operand(N, K, eb, 128)
    xb = f8.dequant_weight(qb, eb)
    qb2, eb2 = f8.quantize_weight_blocks(xb)
    np.testing.assert_array_equal(eb2, eb)
    np.testing.assert_array_equal(f8.e4m3_decode(qb2), f8.e4m3_decode(qb))


def test_gemm_equals_plain_product_on_exact_inputs():
    # products of E4M3 values scaled by powers of two are exact in float64, so
    # the block-scaled product is the plain product of the represented values
    M, N, K = 40, 200, 256
    ea = RNG.integers(-6, 3, (M, K // 128))
    qa = RNG.integers(0, 0x7F, (M, K)).astype(np.uint8)
    eb = RNG.integers(-6, 3, ((N + 127) // 128, K // 128))
    qb = (RNG.integers(0, 0x7F, (N, K)) | 0x80 * RNG.integers(0, 2, (N, K))).astype(np.uint8)
    A = np.zeros((M, K)); B = np.zeros((N, K))
    table = f8.e4m3_decode(ALL)
    for m in range(M):
        for k in range(K):
            A[m, k] = table[qa[m, k]] * 2.0 ** ea[m, k // 128]
    for n in range(N):
        for k in range(K):
            B[n, k] = table[qb[n, k]] * 2.0 ** eb[n // 128, k // 128]
    C = f8.fp8_gemm(qa, ea, qb, eb)
    assert C.shape == (M, N)
    ref = np.array([[sum(A[m, k] * B[n, k] for k in range(K)) for n in range(N)] for m in range(5)])
    np.testing.assert_allclose(C[:5], ref, rtol=1e-12, atol=0)
    np.testing.assert_allclose(C, A @ B.T, rtol=1e-12, atol=0)


def test_weight_block_exponent_is_local():
    # an outlier raises only its own 128 x 128 block's exponent
    w = RNG.standard_normal((300, 384))
    _, e0 = f8.quantize_weight_blocks(w)
    w[200, 300] = 1e4
    _, e1 = f8.quantize_weight_blocks(w)
    diff = np.argwhere(e1 != e0)
    assert diff.tolist() == [[1, 2]]
    assert e0.shape == (3, 3)


# ------------------------------------------------ FP8 prefill (row p, F4) --

def test_fp8_prefill_with_exact_products_is_the_prefill(monkeypatch):
    # the FP8 prefill oracle is the prefill oracle's steps with each
    # projection product replaced by its quantised form: with the product
    # made exact again it must be the float64 prefill itself
    from oracle import fp8_oracle as fo
    import oracle as orc
    from tests.helpers import oracle_cfg, si
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=40, gains="random")
    cfg = oracle_cfg(c, rope="interleaved")
    monkeypatch.setattr(fo, "quantized_product", lambda a, b: np.asarray(a) @ np.asarray(b, dtype=np.float64).T)
    np.testing.assert_allclose(fo.mla_prefill_fp8(cfg, w, x), orc.mla_prefill(cfg, w, x), rtol=1e-12,
                               atol=1e-12)
    w2 = dict(w, kv_norm=np.ones(c["kv_lora_rank"], dtype=np.float32) * 1.5)
    np.testing.assert_allclose(fo.mla_prefill_fp8(cfg, w2, x), orc.mla_prefill(cfg, w2, x), rtol=1e-12,
                               atol=1e-12)


def test_fp8_prefill_quantises_each_projection_input():
    # every product sees quantised operands: the result differs from the
    # exact prefill by an E4M3-sized error (3 mantissa bits: 2^-4 relative
    # per element, averaged down over the reductions), never by more
    from oracle import fp8_oracle as fo
    import oracle as orc
    from tests.helpers import oracle_cfg, row_errors, si
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=64, gains="random")
    cfg = oracle_cfg(c, rope="interleaved")
    rel, _ = row_errors(fo.mla_prefill_fp8(cfg, w, x), orc.mla_prefill(cfg, w, x))
    assert 1e-3 < rel.max() < 0.15, rel.max()
    # the quantised product of one projection is fp8_gemm of the quantised operands
    xa = x.reshape(-1, x.shape[-1]).astype(np.float64)
    qa, ea = fo.quantize_act_tiles(xa)
    qb, eb = fo.quantize_weight_blocks(w["w_down_q"])
    np.testing.assert_array_equal(fo.quantized_product(xa, w["w_down_q"]), fo.fp8_gemm(qa, ea, qb, eb))


def test_fp8_prefill_rows_match_full_fp8_prefill():
    from oracle import fp8_oracle as fo
    from tests.helpers import oracle_cfg, si
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=48, gains="random")
    cfg = oracle_cfg(c, rope="interleaved")
    full = fo.mla_prefill_fp8(cfg, w, x)
    rows = np.array([0, 5, 17, 47])
    yr, lat = fo.mla_prefill_fp8_rows(cfg, w, x, rows, batch=1)
    np.testing.assert_allclose(yr, full[1, rows], rtol=1e-12, atol=1e-12)
    assert lat.shape == (48, c["kv_lora_rank"] + c["qk_rope_head_dim"])
