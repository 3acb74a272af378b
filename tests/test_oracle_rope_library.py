"""Pins of the oracle's YaRN frequencies, YaRN temperature terms and both RoPE
conventions against the DeepSeek-V3 code in the `transformers` library (no GPU).

The RoPE page ("[DeepSeek-V3] Different rotary embedding implementation
between DeepSeek-AI and Transformers", the maintainer's reply and the thread's
summary) points at `modeling_deepseek_v3.py` of `transformers` as the
rotate-half port of DeepSeek-AI's complex (interleaved) rotation, and the
"DeepSeek-V3 Decoupled Implementation" README ("Architecture") gives YaRN with
factor 40 over a 4096-token original context.  These tests tie the oracle's
readings of both to that independent implementation:

* YaRN inverse frequencies (the index-space ramp between the correction dims
  of beta_fast and beta_slow) against `_compute_yarn_parameters`, at the
  long-context V3 parameters and at other parameter sets where an off-by-one
  in the ramp's bounds or denominator would move interior pairs;
* the cos/sin amplitude mscale(f, mscale) / mscale(f, mscale_all_dim) against
  the `attention_factor` that function returns, with mscale != mscale_all_dim;
* the YaRN softmax scale against the attention module's scaling rule;
* the interleaved rotation against `apply_rotary_pos_emb_interleave` (which
  returns its output de-interleaved: equal to ours after the permutation P)
  and the half-split rotation against `apply_rotary_pos_emb` (rotate_half).

`transformers` computes its frequencies in float32, so those comparisons use
a relative bound of 1e-6; the rotations are compared in float64 on both sides.
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc

tf_rope = pytest.importorskip("transformers.modeling_rope_utils")
ds3 = pytest.importorskip("transformers.models.deepseek_v3.modeling_deepseek_v3")
from transformers import DeepseekV3Config  # noqa: E402


def _ds3_config(dr=64, theta=10000.0, factor=40.0, orig=4096, beta_fast=32.0, beta_slow=1.0,
                mscale=1.0, mscale_all_dim=1.0):
    rp = {"rope_type": "yarn", "rope_theta": theta, "factor": factor,
          "original_max_position_embeddings": orig, "beta_fast": beta_fast,
          "beta_slow": beta_slow, "mscale": mscale, "mscale_all_dim": mscale_all_dim}
    cfg = DeepseekV3Config(qk_rope_head_dim=dr, qk_nope_head_dim=128, v_head_dim=128,
                           rope_parameters=rp, max_position_embeddings=int(factor * orig))
    assert cfg.head_dim == dr  # the rotary width transformers derives its dims from
    return cfg


# (d_r, theta, factor, L0, beta_fast, beta_slow): the V3 long-context set,
# then sets whose ramps cover other pair ranges (a few clamp at the ends)
YARN_SETS = [
    (64, 10000.0, 40.0, 4096, 32.0, 1.0),
    (64, 10000.0, 8.0, 4096, 16.0, 2.0),
    (64, 10000.0, 4.0, 2048, 64.0, 4.0),
    (64, 500000.0, 16.0, 8192, 32.0, 1.0),
    (32, 10000.0, 40.0, 4096, 32.0, 1.0),
    (128, 10000.0, 32.0, 4096, 32.0, 1.0),
    (8, 10000.0, 40.0, 4096, 32.0, 1.0),
]


@pytest.mark.parametrize("dr,theta,factor,orig,bf,bs", YARN_SETS)
def test_yarn_inv_freq_matches_transformers(dr, theta, factor, orig, bf, bs):
    cfg = _ds3_config(dr, theta, factor, orig, bf, bs)
    ref, _ = tf_rope._compute_yarn_parameters(cfg)
    ours = orc.yarn_inv_freq(dr, theta, factor, orig, bf, bs)
    np.testing.assert_allclose(ours, ref.double().numpy(), rtol=1e-6, atol=0)


def test_yarn_ramp_interior_v3_pairs_pinned():
    # the interior pairs 11..22 of the V3 set: the library's values, pair by
    # pair; an off-by-one in the ramp (e.g. high - low + 1 in the
    # denominator) moves each of them by a few percent
    cfg = _ds3_config()
    ref = tf_rope._compute_yarn_parameters(cfg)[0].double().numpy()
    ours = orc.yarn_inv_freq(64, 10000.0, 40.0, 4096, 32.0, 1.0)
    np.testing.assert_allclose(ours[11:23], ref[11:23], rtol=1e-6)
    low, high = orc.yarn_correction_range(64, 10000.0, 4096, 32.0, 1.0)
    bad_ramp = np.clip((np.arange(32) - low) / (high - low + 1.0), 0, 1)
    base = orc.rope_inv_freq(64, 10000.0)
    bad = base * (1 - bad_ramp) + base / 40.0 * bad_ramp
    assert np.abs(bad[11:23] / ref[11:23] - 1).max() > 1e-2


@pytest.mark.parametrize("factor,mscale,mscale_all_dim", [
    (40.0, 1.0, 1.0), (40.0, 0.707, 0.707), (40.0, 0.8, 1.2), (8.0, 1.0, 0.5), (4.0, 1.5, 1.0)])
def test_yarn_amplitude_and_mscale_match_transformers(factor, mscale, mscale_all_dim):
    cfg = _ds3_config(factor=factor, mscale=mscale, mscale_all_dim=mscale_all_dim)
    _, attention_factor = tf_rope._compute_yarn_parameters(cfg)
    ocfg = orc.Cfg(7168, 128, 1536, 512, 128, 64, 128, rope_factor=factor, mscale=mscale,
                   mscale_all_dim=mscale_all_dim)
    assert orc.cfg_cos_sin_scale(ocfg) == pytest.approx(attention_factor, rel=1e-12)
    for m in (mscale, mscale_all_dim):
        assert orc.yarn_mscale(factor, m) == pytest.approx(ds3.yarn_get_mscale(factor, m),
                                                          rel=1e-15)
    assert orc.yarn_mscale(1.0, mscale) == ds3.yarn_get_mscale(1.0, mscale) == 1.0


@pytest.mark.parametrize("factor,mscale_all_dim", [(40.0, 1.0), (40.0, 0.707), (8.0, 1.3)])
def test_yarn_softmax_scale_matches_transformers(factor, mscale_all_dim):
    # the attention module's scaling: (d_n + d_r)^-1/2, times
    # mscale(factor, mscale_all_dim)^2 under YaRN
    cfg = _ds3_config(factor=factor, mscale_all_dim=mscale_all_dim)
    ref = ds3.yarn_apply_mscale(cfg.rope_parameters, (128 + 64) ** -0.5)
    ocfg = orc.Cfg(7168, 128, 1536, 512, 128, 64, 128, rope_factor=factor,
                   mscale_all_dim=mscale_all_dim)
    assert orc.softmax_scale(ocfg) == pytest.approx(ref, rel=1e-12)


def test_yarn_rotary_embedding_cos_sin_match_transformers():
    # the whole cos/sin table the DeepSeek-V3 rotary module produces (float32)
    # at small positions, amplitude included (mscale != mscale_all_dim)
    cfg = _ds3_config(factor=40.0, mscale=0.9, mscale_all_dim=1.1)
    rot = ds3.DeepseekV3RotaryEmbedding(cfg)
    pos = torch.arange(0, 256, dtype=torch.long)[None]
    cos, sin = rot(torch.zeros(1, dtype=torch.float32), pos)
    ocfg = orc.Cfg(7168, 128, 1536, 512, 128, 64, 128, rope_factor=40.0, mscale=0.9,
                   mscale_all_dim=1.1)
    c, s = orc.rope_cos_sin(np.arange(256), orc.cfg_inv_freq(ocfg), orc.cfg_cos_sin_scale(ocfg))
    # transformers lays cos/sin out as cat(freqs, freqs)
    np.testing.assert_allclose(cos[0, :, :32].double().numpy(), c, atol=2e-5)
    np.testing.assert_allclose(cos[0, :, 32:].double().numpy(), c, atol=2e-5)
    np.testing.assert_allclose(sin[0, :, :32].double().numpy(), s, atol=2e-5)


def _angles(n, d, seed):
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, 40000, size=n)
    inv = orc.yarn_inv_freq(d, 10000.0, 40.0, 4096, 32.0, 1.0)
    c, s = orc.rope_cos_sin(pos, inv)
    return pos, c, s


@pytest.mark.parametrize("d", [8, 64])
def test_interleaved_rope_matches_transformers_after_deinterleave(d):
    # transformers' interleaved rotation returns cat(even-rotated, odd-rotated):
    # our interleaved output (layout kept) read through P
    rng = np.random.default_rng(31)
    n, H = 40, 3
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((n, 1, d))
    pos, c, s = _angles(n, d, 32)
    cc = torch.from_numpy(np.concatenate([c, c], axis=-1))[None]  # [1, n, d]
    ss = torch.from_numpy(np.concatenate([s, s], axis=-1))[None]
    # transformers' layout [batch, heads, seq, d]
    qt = torch.from_numpy(q.transpose(1, 0, 2))[None]
    kt = torch.from_numpy(k.transpose(1, 0, 2))[None]
    qr, kr = ds3.apply_rotary_pos_emb_interleave(qt, kt, cc, ss)
    qr = qr[0].numpy().transpose(1, 0, 2)
    kr = kr[0].numpy().transpose(1, 0, 2)
    P = orc.deinterleave_perm(d)
    np.testing.assert_allclose(orc.rope_interleaved(q, c, s)[..., P], qr, rtol=0, atol=1e-14)
    np.testing.assert_allclose(orc.rope_interleaved(k, c, s)[..., P], kr, rtol=0, atol=1e-14)
    # scores agree without any permutation (both sides permute alike)
    ours = np.einsum("thd,tgd->thg", orc.rope_interleaved(q, c, s), orc.rope_interleaved(k, c, s))
    theirs = np.einsum("thd,tgd->thg", qr, kr)
    np.testing.assert_allclose(ours, theirs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [8, 64])
def test_half_split_rope_matches_transformers_rotate_half(d):
    rng = np.random.default_rng(33)
    n, H = 40, 3
    q = rng.standard_normal((n, H, d))
    k = rng.standard_normal((n, 1, d))
    pos, c, s = _angles(n, d, 34)
    cc = torch.from_numpy(np.concatenate([c, c], axis=-1))[None]
    ss = torch.from_numpy(np.concatenate([s, s], axis=-1))[None]
    qt = torch.from_numpy(q.transpose(1, 0, 2))[None]
    kt = torch.from_numpy(k.transpose(1, 0, 2))[None]
    qr, kr = ds3.apply_rotary_pos_emb(qt, kt, cc, ss)
    np.testing.assert_allclose(orc.rope_half_split(q, c, s), qr[0].numpy().transpose(1, 0, 2),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(orc.rope_half_split(k, c, s), kr[0].numpy().transpose(1, 0, 2),
                               rtol=0, atol=1e-14)


def test_conventions_differ_on_same_input_like_the_issue():
    # the issue's observation: fed the same q_pe / k_pe, the two formulations
    # give different scores between tokens at different positions (permuting
    # the weights is what makes them agree); at the issue's width 64
    rng = np.random.default_rng(35)
    q = rng.standard_normal((16, 1, 64))
    k = rng.standard_normal((16, 1, 64))
    pos, c, s = _angles(16, 64, 36)

    def scores(rope, qq, kk):
        return np.einsum("thd,ugd->tu", rope(qq, c, s), rope(kk, c, s))

    a = scores(orc.rope_interleaved, q, k)
    b = scores(orc.rope_half_split, q, k)
    assert np.abs(a - b).max() > 1e-1
    P = orc.deinterleave_perm(64)
    np.testing.assert_allclose(a, scores(orc.rope_half_split, q[..., P], k[..., P]),
                               rtol=1e-12, atol=1e-12)
    assert math.isfinite(float(a.sum()))
