"""Pins of the oracle's RoPE, YaRN and RMSNorm against what the pages and the
mathematics fix (no GPU)."""

import math

import numpy as np
import pytest
import torch

import oracle as orc
from tests.helpers import oracle_cfg, si

RNG = np.random.default_rng(11)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
@pytest.mark.parametrize("d", [2, 8, 32, 64])
def test_rope_preserves_pair_norms(conv, d):
    # a rotation keeps the length of each rotated pair
    x = RNG.standard_normal((50, 3, d))
    pos = RNG.integers(0, 40000, size=50)
    cfg = orc.Cfg(64, 3, 8, 8, 8, d, 8, rope_convention=conv)
    y = orc.apply_rope(x, pos, cfg)
    h = d // 2
    if conv == "half_split":
        nx = x[..., :h] ** 2 + x[..., h:] ** 2
        ny = y[..., :h] ** 2 + y[..., h:] ** 2
    else:
        nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_rope_position_zero_is_identity(conv):
    x = RNG.standard_normal((1, 4, 64))
    cfg = orc.Cfg(64, 4, 8, 8, 8, 64, 8, rope_convention=conv)
    np.testing.assert_array_equal(orc.apply_rope(x, [0], cfg), x)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_rope_relative_position(conv):
    # <R(p+D) q, R(m+D) k> = <R(p) q, R(m) k>: scores depend on p - m only
    cfg = orc.Cfg(64, 1, 8, 8, 8, 64, 8, rope_convention=conv)
    q = RNG.standard_normal((1, 64))
    k = RNG.standard_normal((1, 64))
    for p, m, delta in [(5, 3, 100), (1000, 7, 17), (0, 0, 4095)]:
        a = orc.apply_rope(q, [p + delta], cfg) @ orc.apply_rope(k, [m + delta], cfg).T
        b = orc.apply_rope(q, [p], cfg) @ orc.apply_rope(k, [m], cfg).T
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_rope_d2_conventions_coincide():
    # with a single pair both conventions rotate (x0, x1) the same way
    x = RNG.standard_normal((30, 2))
    pos = np.arange(30) * 37
    a = orc.apply_rope(x, pos, orc.Cfg(64, 1, 8, 8, 8, 2, 8, rope_convention="half_split"))
    b = orc.apply_rope(x, pos, orc.Cfg(64, 1, 8, 8, 8, 2, 8, rope_convention="interleaved"))
    np.testing.assert_array_equal(a, b)


def test_interleaved_is_complex_multiplication():
    # the complex formulation: (x_2i + i x_2i+1) * exp(i p inv_freq_i)
    d = 64
    x = RNG.standard_normal((40, 5, d))
    pos = RNG.integers(0, 5000, size=40)
    cfg = orc.Cfg(64, 5, 8, 8, 8, d, 8, rope_convention="interleaved")
    z = x[..., 0::2] + 1j * x[..., 1::2]
    inv = 10000.0 ** (-np.arange(0, d, 2) / d)
    z = z * np.exp(1j * pos[:, None, None] * inv[None, None, :])
    ref = np.empty_like(x)
    ref[..., 0::2] = z.real
    ref[..., 1::2] = z.imag
    np.testing.assert_allclose(orc.apply_rope(x, pos, cfg), ref, rtol=1e-12, atol=1e-12)


def test_half_split_is_complex_multiplication_of_halves():
    # rotate-half: (x_i + i x_{i+d/2}) * exp(i p inv_freq_i)
    d = 32
    x = RNG.standard_normal((20, 3, d))
    pos = RNG.integers(0, 5000, size=20)
    cfg = orc.Cfg(64, 3, 8, 8, 8, d, 8, rope_convention="half_split")
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(
        1j * pos[:, None, None] * (10000.0 ** (-np.arange(0, d, 2) / d))[None, None])
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(orc.apply_rope(x, pos, cfg), ref, rtol=1e-12, atol=1e-12)


def test_rope_basis_vector_closed_form():
    # e_0 at position p, rotate-half: (cos p, 0, .., sin p, 0, ..) since
    # inv_freq_0 = 1; e_1 turns by p * theta^(-2/d)
    d = 8
    cfg = orc.Cfg(64, 1, 8, 8, 8, d, 8, rope_convention="half_split")
    for p in (1, 3, 100):
        e0 = np.zeros((1, d)); e0[0, 0] = 1
        y = orc.apply_rope(e0, [p], cfg)[0]
        assert y[0] == pytest.approx(math.cos(p), abs=1e-15)
        assert y[d // 2] == pytest.approx(math.sin(p), abs=1e-15)
        e1 = np.zeros((1, d)); e1[0, 1] = 1
        y = orc.apply_rope(e1, [p], cfg)[0]
        a = p * 10000.0 ** (-2.0 / d)
        assert y[1] == pytest.approx(math.cos(a), abs=1e-15)
        assert y[d // 2 + 1] == pytest.approx(math.sin(a), abs=1e-15)


@pytest.mark.parametrize("d", [8, 32, 64])
def test_conventions_equal_up_to_deinterleave_permutation(d):
    # IL(x) = P^-1 HS(P x), exactly (same products, same order)
    x = RNG.standard_normal((64, 7, d))
    pos = RNG.integers(0, 40000, size=64)
    hs = orc.Cfg(64, 7, 8, 8, 8, d, 8, rope_convention="half_split")
    il = orc.Cfg(64, 7, 8, 8, 8, d, 8, rope_convention="interleaved")
    P = orc.deinterleave_perm(d)
    Pinv = np.argsort(P)
    lhs = orc.apply_rope(x, pos, il)
    rhs = orc.apply_rope(x[..., P], pos, hs)[..., Pinv]
    np.testing.assert_array_equal(lhs, rhs)


def test_deinterleave_perm_definition():
    P = orc.deinterleave_perm(8)
    x = np.arange(8.0)
    np.testing.assert_array_equal(x[P], [0, 2, 4, 6, 1, 3, 5, 7])


def test_conventions_differ_on_same_input():
    # on identical q_pe the two formulations are not the same function
    d = 64
    x = RNG.standard_normal((16, 4, d))
    pos = np.arange(16)
    a = orc.apply_rope(x, pos, orc.Cfg(64, 4, 8, 8, 8, d, 8, rope_convention="half_split"))
    b = orc.apply_rope(x, pos, orc.Cfg(64, 4, 8, 8, 8, d, 8, rope_convention="interleaved"))
    np.testing.assert_array_equal(a[0], b[0])  # position 0: both identity
    assert np.abs(a[1:] - b[1:]).max() > 0.1


# ------------------------------------------------------------------ YaRN ---

def test_yarn_factor_one_is_plain_rope():
    np.testing.assert_array_equal(
        orc.yarn_inv_freq(64, 10000.0, 1.0, 4096, 32, 1),
        orc.rope_inv_freq(64, 10000.0))
    assert orc.yarn_mscale(1.0, 1.0) == 1.0


def test_yarn_v3_boundaries():
    # factor 40 over an original 4096 context: 40 * 4096 = 163,840 tokens,
    # the context the V3 README states.  Correction pair indices derived by
    # hand: 64 ln(4096 / (2 pi 32)) / (2 ln 1e4) = 10.47 -> floor 10 and
    # 64 ln(4096 / (2 pi)) / (2 ln 1e4) = 22.51 -> ceil 23.
    c = si.CONFIGS["v3_yarn"]
    assert c["rope_factor"] * c["original_max_position_embeddings"] == 163840
    low, high = orc.yarn_correction_range(64, 10000.0, 4096, 32.0, 1.0)
    assert (low, high) == (10, 23)
    base = orc.rope_inv_freq(64, 10000.0)
    yf = orc.yarn_inv_freq(64, 10000.0, 40.0, 4096, 32.0, 1.0)
    np.testing.assert_array_equal(yf[:11], base[:11])
    np.testing.assert_allclose(yf[23:], base[23:] / 40.0, rtol=1e-15)
    # in between: strictly between the two, interpolating monotonically
    r = yf[11:23] / base[11:23]
    assert np.all(r < 1) and np.all(r > 1 / 40.0) and np.all(np.diff(r) < 0)


def test_yarn_softmax_scale_v3():
    # 0.1 ln 40 + 1 = 1.368888 (mscale_all_dim 1), squared = 1.873854;
    # the base scale 1/sqrt(128 + 64) is the MLA listing's 1/sqrt(dk)
    cfg = oracle_cfg(si.CONFIGS["v3_yarn"])
    assert orc.yarn_mscale(40.0, 1.0) == pytest.approx(1.368888, abs=1e-6)
    assert orc.softmax_scale(cfg) == pytest.approx(0.135234, abs=1e-6)
    assert orc.softmax_scale(oracle_cfg(si.CONFIGS["v3_prefill"])) == pytest.approx(
        1 / math.sqrt(192), rel=1e-15)


# --------------------------------------------------------------- RMSNorm ---

def test_rmsnorm_unit_rms_and_scale_invariance():
    x = RNG.standard_normal((20, 1536)) * 3.0
    g = np.ones(1536)
    y = orc.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rmsnorm(5.0 * x, g, 0.0), y, rtol=1e-13)
    # eps enters inside the root: for x = 0 rows the output is exactly zero
    assert np.all(orc.rmsnorm(np.zeros((2, 8)), np.ones(8), 1e-6) == 0)


def test_rmsnorm_matches_torch_library():
    x = RNG.standard_normal((10, 256))
    g = 1.0 + 0.1 * RNG.standard_normal(256)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,),
                                       torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(orc.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)
