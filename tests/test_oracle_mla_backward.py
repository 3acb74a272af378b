"""Pins of the MLA backward oracle (oracle/mla_backward_oracle.py), no GPU.

The gradients of L = <dy, MLA(x)> are checked against what fixes them
independently of the chain rule as written there:

* central finite differences of L in x and in sampled elements of every
  weight (the pages' own check of the reference's gradients, "DSV3 Native
  PyTorch Reference", section "NumPy Oracle": full-parameter finite
  differences on a micro configuration), float64, both RoPE conventions,
  YaRN, with and without the RMSNorm on c_kv;
* torch float64 autograd of a forward written here with torch ops (its own
  RoPE, norm and masked softmax), on the small configuration;
* the shared RoPE key: its weight's gradient is the sum over heads, so with
  the heads made identical the gradient scales with the head count."""

import numpy as np
import pytest
import torch

import oracle as orc
from oracle.mla_backward_oracle import mla_backward
from tests.helpers import oracle_cfg, shrink, si


def _loss(cfg, w, x, dy):
    return float(np.sum(orc.mla_prefill(cfg, w, x) * dy))


def _case(conv="half_split", yarn=False, kv_norm=False, S=6, B=2, seed=71):
    c = shrink(si.CONFIGS["tiny"], rope=conv, seed=seed)
    if yarn:
        c = shrink(c, rope_factor=8.0, original_max_position_embeddings=4, beta_fast=2.0, beta_slow=1.0,
                   mscale=0.9, mscale_all_dim=1.1)
    x, w = si.make_inputs(c, seq=S, batch=B, gains="random")
    x = x.astype(np.float64)
    w = {k: v.astype(np.float64) * (3.0 if k.startswith("w_") else 1.0) for k, v in w.items()}
    rng = np.random.default_rng(seed + 1)
    if kv_norm:
        w["kv_norm"] = 1.0 + 0.2 * rng.standard_normal(c["kv_lora_rank"])
    dy = rng.standard_normal(x.shape)
    return oracle_cfg(c), w, x, dy


@pytest.mark.parametrize("conv,yarn,kv_norm", [("half_split", False, False), ("interleaved", False, True),
                                               ("interleaved", True, False)])
def test_backward_matches_finite_differences(conv, yarn, kv_norm):
    cfg, w, x, dy = _case(conv, yarn, kv_norm)
    dx, g = mla_backward(cfg, w, x, dy)
    h = 1e-6
    rng = np.random.default_rng(5)
    # x: every element of one token row and a few others
    idx = [(1, 3, j) for j in range(x.shape[2])] + [tuple(rng.integers(0, n) for n in x.shape) for _ in range(8)]
    for i in idx:
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        fd = (_loss(cfg, w, xp, dy) - _loss(cfg, w, xm, dy)) / (2 * h)
        assert abs(fd - dx[i]) <= 1e-6 * max(1.0, abs(fd)), (i, fd, dx[i])
    for name, W in w.items():
        flat = W.reshape(-1)
        for k in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            wp, wm = dict(w), dict(w)
            wp[name] = flat.copy()
            wp[name][k] += h
            wp[name] = wp[name].reshape(W.shape)
            wm[name] = flat.copy()
            wm[name][k] -= h
            wm[name] = wm[name].reshape(W.shape)
            fd = (_loss(cfg, wp, x, dy) - _loss(cfg, wm, x, dy)) / (2 * h)
            got = g[name].reshape(-1)[k]
            assert abs(fd - got) <= 1e-6 * max(1.0, abs(fd)), (name, k, fd, got)
    assert set(g) == set(w)


def _torch_forward(cfg, tw, tx):
    """The MLA forward in torch ops (float64), written independently of the
    oracle: its own RMSNorm, rotation and masked softmax."""
    B, S, D = tx.shape
    H, dn, dr, dv = (cfg.num_attention_heads, cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.v_head_dim)

    def norm(t, g):
        return t * torch.rsqrt((t * t).mean(-1, keepdim=True) + cfg.rms_norm_eps) * g

    inv = torch.tensor(orc.cfg_inv_freq(cfg))
    amp = orc.cfg_cos_sin_scale(cfg)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * inv[None]
    cos, sin = torch.cos(ang) * amp, torch.sin(ang) * amp

    def rope(t):  # t [B, S, ..., dr]
        shp = (1, S) + (1,) * (t.dim() - 3) + (dr // 2,)
        c, s_ = cos.reshape(shp), sin.reshape(shp)
        if cfg.rope_convention == "half_split":
            a, b = t[..., :dr // 2], t[..., dr // 2:]
            return torch.cat([a * c - b * s_, b * c + a * s_], -1)
        a, b = t[..., 0::2], t[..., 1::2]
        return torch.stack([a * c - b * s_, b * c + a * s_], -1).reshape(t.shape)

    c_qn = norm(tx @ tw["w_down_q"].T, tw["q_norm"])
    c_kv = tx @ tw["w_down_kv"].T
    if "kv_norm" in tw:
        c_kv = norm(c_kv, tw["kv_norm"])
    q = torch.cat([(c_qn @ tw["w_up_q"].T).reshape(B, S, H, dn),
                   rope((c_qn @ tw["w_qr"].T).reshape(B, S, H, dr))], -1)
    k_pe = rope(tx @ tw["w_kr"].T)  # [B, S, dr]
    k = torch.cat([(c_kv @ tw["w_up_k"].T).reshape(B, S, H, dn), k_pe[:, :, None].expand(B, S, H, dr)], -1)
    v = (c_kv @ tw["w_up_v"].T).reshape(B, S, H, dv)
    s = torch.einsum("bihd,bjhd->bhij", q, k) * orc.softmax_scale(cfg)
    s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, -1), v).reshape(B, S, H * dv)
    return o @ tw["wo"].T


@pytest.mark.parametrize("conv,kv_norm", [("interleaved", False), ("half_split", True)])
def test_backward_matches_torch_autograd(conv, kv_norm):
    c = shrink(si.CONFIGS["small"], rope=conv)
    x, w = si.make_inputs(c, seq=40, batch=2, gains="random")
    w = {k: v.astype(np.float64) for k, v in w.items()}
    if kv_norm:
        w["kv_norm"] = 1.0 + 0.1 * np.random.default_rng(3).standard_normal(c["kv_lora_rank"])
    cfg = oracle_cfg(c)
    dy = np.random.default_rng(4).standard_normal((2, 40, c["hidden_size"]))
    dx, g = mla_backward(cfg, w, x, dy)
    tw = {k: torch.tensor(v, requires_grad=True) for k, v in w.items()}
    tx = torch.tensor(x.astype(np.float64), requires_grad=True)
    y = _torch_forward(cfg, tw, tx)
    np.testing.assert_allclose(y.detach().numpy(), orc.mla_prefill(cfg, w, x), rtol=1e-10, atol=1e-12)
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-9, atol=1e-11)
    for k in w:
        np.testing.assert_allclose(g[k], tw[k].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=k)


def test_shared_rope_key_gradient_sums_heads():
    # with every head's weights identical (w_o's head columns tiled), the
    # loss is H times the one-head loss, each head contributing the same
    # k_pe gradient: dW_kr is H times the one-head gradient (a gradient
    # taken from one head only would give 1x)
    c = shrink(si.CONFIGS["tiny"], num_attention_heads=1, seed=91)
    x, w = si.make_inputs(c, seq=5, batch=1, gains="random")
    w = {k: v.astype(np.float64) for k, v in w.items()}
    cfg1 = oracle_cfg(c)
    dy = np.random.default_rng(92).standard_normal(x.shape)
    H = 4
    wH = dict(w)
    for name in ("w_up_q", "w_qr", "w_up_k", "w_up_v"):
        wH[name] = np.tile(w[name], (H, 1))
    wH["wo"] = np.tile(w["wo"], (1, H))
    cfgH = oracle_cfg(shrink(c, num_attention_heads=H))
    _, g1 = mla_backward(cfg1, w, x, dy)
    _, gH = mla_backward(cfgH, wH, x, dy)
    np.testing.assert_allclose(gH["w_kr"], H * g1["w_kr"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gH["w_down_kv"], H * g1["w_down_kv"], rtol=1e-10, atol=1e-13)
