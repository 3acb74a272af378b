"""Pins of the oracle's MLA prefill and decode (no GPU).

Each test checks the oracle against something other than itself: loop-level
brute force on tiny shapes, PyTorch's own float64 library routines, closed
forms (one token, zero query weights), invariants the pages state
(causality; the two RoPE conventions agreeing once the weights are permuted)
and the algebraic identity of absorbed and expanded decode."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc
from tests.helpers import oracle_cfg, shrink, si

TINY = si.CONFIGS["tiny"]


def _tiny_inputs(conv="half_split", gains="random", S=None, B=None):
    c = shrink(TINY, rope=conv)
    x, w = si.make_inputs(c, seq=S, batch=B, gains=gains)
    return oracle_cfg(c), x.astype(np.float64), {k: v.astype(np.float64) for k, v in w.items()}


def _brute_force_prefill(cfg, w, x):
    """Scalar loops over tokens, heads and channels with math.* only."""
    B, S, D = x.shape
    H, dn, dr, dv = (cfg.num_attention_heads, cfg.qk_nope_head_dim,
                     cfg.qk_rope_head_dim, cfg.v_head_dim)
    rq, rkv = cfg.q_lora_rank, cfg.kv_lora_rank

    def lin(W, vec):
        return [sum(W[o][i] * vec[i] for i in range(len(vec))) for o in range(len(W))]

    def rope(vec, p):
        h = dr // 2
        out = list(vec)
        for i in range(h):
            a = p * cfg.rope_theta ** (-2.0 * i / dr)
            if cfg.rope_convention == "half_split":
                u, v = vec[i], vec[i + h]
                out[i] = u * math.cos(a) - v * math.sin(a)
                out[i + h] = v * math.cos(a) + u * math.sin(a)
            else:
                u, v = vec[2 * i], vec[2 * i + 1]
                out[2 * i] = u * math.cos(a) - v * math.sin(a)
                out[2 * i + 1] = v * math.cos(a) + u * math.sin(a)
        return out

    Wl = {k: v.tolist() for k, v in w.items()}
    y = np.zeros((B, S, D))
    for b in range(B):
        toks = []
        for s in range(S):
            xs = x[b, s].tolist()
            cq = lin(Wl["w_down_q"], xs)
            ms = sum(t * t for t in cq) / rq
            cqn = [cq[i] / math.sqrt(ms + cfg.rms_norm_eps) * Wl["q_norm"][i] for i in range(rq)]
            qn = lin(Wl["w_up_q"], cqn)
            qp = lin(Wl["w_qr"], cqn)
            ckv = lin(Wl["w_down_kv"], xs)
            kp = rope(lin(Wl["w_kr"], xs), s)
            kn = lin(Wl["w_up_k"], ckv)
            vv = lin(Wl["w_up_v"], ckv)
            toks.append(dict(
                q=[qn[h * dn:(h + 1) * dn] + rope(qp[h * dr:(h + 1) * dr], s) for h in range(H)],
                k=[kn[h * dn:(h + 1) * dn] + kp for h in range(H)],
                v=[vv[h * dv:(h + 1) * dv] for h in range(H)]))
        for s in range(S):
            o = []
            for h in range(H):
                q = toks[s]["q"][h]
                sc = [sum(q[c] * toks[j]["k"][h][c] for c in range(dn + dr)) /
                      math.sqrt(dn + dr) for j in range(s + 1)]
                m = max(sc)
                e = [math.exp(t - m) for t in sc]
                z = sum(e)
                o += [sum(e[j] / z * toks[j]["v"][h][c] for j in range(s + 1)) for c in range(dv)]
            y[b, s] = lin(Wl["wo"], o)
    return y


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_prefill_matches_brute_force(conv):
    cfg, x, w = _tiny_inputs(conv, S=6, B=2)
    np.testing.assert_allclose(orc.mla_prefill(cfg, w, x), _brute_force_prefill(cfg, w, x),
                               rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_varlen_prefill_is_per_sequence_brute_force(conv):
    # packed sequences of lengths 3, 0, 5, 1: each block of rows is the
    # brute-force forward of that sequence alone (positions from 0)
    cfg, x, w = _tiny_inputs(conv, S=9, B=1)
    lens = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, lat = orc.mla_prefill_varlen(cfg, w, x[0], cu)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        a = cu[b]
        ref = _brute_force_prefill(cfg, w, x[:, a:a + L])[0]
        np.testing.assert_allclose(y[a:a + L], ref, rtol=1e-10, atol=1e-13)
    # latent rows: c_kv then the post-RoPE k_pe of each token at its own position
    _, inter = orc.mla_prefill(cfg, w, x[:, 3:8], want_intermediates=True)
    np.testing.assert_allclose(lat[3:8], np.concatenate([inter["c_kv"][0], inter["k_pe"][0]], -1),
                               rtol=1e-12, atol=1e-14)


def test_varlen_prefill_order_and_independence():
    # reordering the sequences reorders the output blocks; changing one
    # sequence's tokens leaves every other sequence's rows unchanged
    cfg, x, w = _tiny_inputs("interleaved", S=12, B=1)
    x = x[0]
    y, _ = orc.mla_prefill_varlen(cfg, w, x, [0, 5, 12])
    y_sw, _ = orc.mla_prefill_varlen(cfg, w, np.concatenate([x[5:], x[:5]]), [0, 7, 12])
    np.testing.assert_allclose(y_sw[:7], y[5:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y_sw[7:], y[:5], rtol=1e-12, atol=1e-14)
    x2 = x.copy()
    x2[6] += 1.0
    y2, _ = orc.mla_prefill_varlen(cfg, w, x2, [0, 5, 12])
    assert np.array_equal(y2[:5], y[:5]) and not np.allclose(y2[5:], y[5:])


def _torch_library_prefill(cfg, w, x):
    """The same forward built from PyTorch float64 library routines: linear,
    rms_norm, complex multiplication for RoPE, causal SDPA."""
    t = {k: torch.from_numpy(v) for k, v in w.items()}
    xt = torch.from_numpy(x)
    B, S, _ = x.shape
    H, dn, dr, dv = (cfg.num_attention_heads, cfg.qk_nope_head_dim,
                     cfg.qk_rope_head_dim, cfg.v_head_dim)
    inv = cfg.rope_theta ** (-torch.arange(0, dr, 2, dtype=torch.float64) / dr)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * inv[None]
    rot = torch.polar(torch.ones_like(ang), ang)  # [S, dr/2]

    def rope(v):  # v [..., S, dr]
        if cfg.rope_convention == "interleaved":
            z = torch.view_as_complex(v.reshape(*v.shape[:-1], dr // 2, 2).contiguous()) * rot
            return torch.view_as_real(z).reshape(v.shape)
        z = torch.complex(v[..., : dr // 2], v[..., dr // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    cq = F.rms_norm(F.linear(xt, t["w_down_q"]), (cfg.q_lora_rank,), t["q_norm"],
                    eps=cfg.rms_norm_eps)
    qn = F.linear(cq, t["w_up_q"]).view(B, S, H, dn).transpose(1, 2)
    qp = rope(F.linear(cq, t["w_qr"]).view(B, S, H, dr).transpose(1, 2))
    ckv = F.linear(xt, t["w_down_kv"])
    kp = rope(F.linear(xt, t["w_kr"]))[:, None].expand(B, H, S, dr)
    kn = F.linear(ckv, t["w_up_k"]).view(B, S, H, dn).transpose(1, 2)
    v = F.linear(ckv, t["w_up_v"]).view(B, S, H, dv).transpose(1, 2)
    o = F.scaled_dot_product_attention(torch.cat([qn, qp], -1), torch.cat([kn, kp], -1), v,
                                       is_causal=True, scale=orc.softmax_scale(cfg))
    return F.linear(o.transpose(1, 2).reshape(B, S, H * dv), t["wo"]).numpy()


@pytest.mark.parametrize("name,conv,S", [("tiny", "half_split", 16), ("tiny", "interleaved", 16),
                                          ("small", "half_split", 64), ("small", "interleaved", 64)])
def test_prefill_matches_torch_library(name, conv, S):
    c = shrink(si.CONFIGS[name], rope=conv)
    x, w = si.make_inputs(c, seq=S, gains="random")
    cfg = oracle_cfg(c)
    x = x.astype(np.float64)
    w = {k: v.astype(np.float64) for k, v in w.items()}
    np.testing.assert_allclose(orc.mla_prefill(cfg, w, x), _torch_library_prefill(cfg, w, x),
                               rtol=1e-9, atol=1e-12)


def test_single_token_closed_form():
    # S = 1: softmax over one key is 1, so o_h = V_0 = W_uv_h c_kv and
    # y = wo (concat_h W_uv_h c_kv), whatever the query side does
    cfg, x, w = _tiny_inputs(S=1)
    ckv = x[0, 0] @ w["w_down_kv"].T
    ref = (w["w_up_v"] @ ckv) @ w["wo"].T
    np.testing.assert_allclose(orc.mla_prefill(cfg, w, x)[0, 0], ref, rtol=1e-12)


def test_zero_query_weights_give_cumulative_mean():
    # W_uq = W_qr = 0: all scores 0, softmax uniform over j <= i,
    # so o_i is the running mean of V_0..V_i
    cfg, x, w = _tiny_inputs()
    w["w_up_q"][:] = 0
    w["w_qr"][:] = 0
    _, inter = orc.mla_prefill(cfg, w, x, want_intermediates=True)
    v = inter["v"][0]  # [S, H, dv]
    cm = np.cumsum(v, axis=0) / np.arange(1, v.shape[0] + 1)[:, None, None]
    np.testing.assert_allclose(inter["o"][0], cm.reshape(v.shape[0], -1), rtol=1e-12, atol=1e-15)


def test_causality_future_tokens_do_not_leak():
    cfg, x, w = _tiny_inputs(S=16)
    y0 = orc.mla_prefill(cfg, w, x)
    x2 = x.copy()
    x2[:, 9:] = np.random.default_rng(5).standard_normal(x2[:, 9:].shape) * 7
    y1 = orc.mla_prefill(cfg, w, x2)
    np.testing.assert_array_equal(y1[:, :9], y0[:, :9])
    assert np.abs(y1[:, 9:] - y0[:, 9:]).max() > 1e-3


def test_batch_independence():
    cfg, x, w = _tiny_inputs(B=3)
    y = orc.mla_prefill(cfg, w, x)
    np.testing.assert_allclose(orc.mla_prefill(cfg, w, x[1:2])[0], y[1], rtol=1e-13, atol=1e-15)


def test_head_permutation_equivariance():
    # permuting the heads consistently in every per-head weight leaves y unchanged
    cfg, x, w = _tiny_inputs()
    H, dn, dr, dv = 4, 16, 8, 16
    perm = np.array([2, 0, 3, 1])

    def rows(W, d):
        return W.reshape(H, d, -1)[perm].reshape(H * d, -1)

    w2 = dict(w)
    w2["w_up_q"] = rows(w["w_up_q"], dn)
    w2["w_qr"] = rows(w["w_qr"], dr)
    w2["w_up_k"] = rows(w["w_up_k"], dn)
    w2["w_up_v"] = rows(w["w_up_v"], dv)
    w2["wo"] = w["wo"].reshape(-1, H, dv)[:, perm].reshape(-1, H * dv)
    np.testing.assert_allclose(orc.mla_prefill(cfg, w2, x), orc.mla_prefill(cfg, w, x),
                               rtol=1e-12, atol=1e-15)


def test_attention_core_matches_sdpa():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 37, 24))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (q, k, v)),
                                         is_causal=True, scale=0.3)[0].numpy()
    np.testing.assert_allclose(orc.causal_attention(q, k, v, 0.3), ref, rtol=1e-12, atol=1e-14)


def _permute_for_half_split(cfg, w):
    """Weights that make the rotate-half convention reproduce the interleaved
    one: rows of w_qr (per head) and w_kr reordered by the even/odd
    de-interleave of the rope columns."""
    H, dr = cfg.num_attention_heads, cfg.qk_rope_head_dim
    P = orc.deinterleave_perm(dr)
    w2 = dict(w)
    w2["w_qr"] = w["w_qr"].reshape(H, dr, -1)[:, P].reshape(H * dr, -1)
    w2["w_kr"] = w["w_kr"][P]
    return w2


@pytest.mark.parametrize("name,S", [("tiny", 16), ("small", 64)])
def test_conventions_agree_after_weight_permutation(name, S):
    c = si.CONFIGS[name]
    x, w = si.make_inputs(c, seq=S)
    x = x.astype(np.float64)
    w = {k: v.astype(np.float64) for k, v in w.items()}
    il = oracle_cfg(c, rope="interleaved")
    hs = oracle_cfg(c, rope="half_split")
    y_il = orc.mla_prefill(il, w, x)
    y_hs_perm = orc.mla_prefill(hs, _permute_for_half_split(il, w), x)
    y_hs_same = orc.mla_prefill(hs, w, x)
    np.testing.assert_allclose(y_hs_perm, y_il, rtol=1e-10, atol=1e-13)
    # and without the permutation the two differ
    assert np.abs(y_hs_same - y_il).max() > 1e-3 * np.abs(y_il).max()


def test_prefill_rows_match_full_prefill():
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=96, gains="random")
    cfg = oracle_cfg(c, rope="interleaved")
    y, inter = orc.mla_prefill(cfg, w, x, want_intermediates=True)
    rows = np.array([0, 5, 31, 95])
    yr, lat = orc.mla_prefill_rows(cfg, w, x, rows, batch=1)
    np.testing.assert_allclose(yr, y[1, rows], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lat[:, :128], inter["c_kv"][1], rtol=1e-13)
    np.testing.assert_allclose(lat[:, 128:], inter["k_pe"][1], rtol=1e-13)


# ---------------------------------------------------------------- decode ---

@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_absorbed_decode_equals_expanded(conv):
    c = shrink(si.CONFIGS["small"], rope=conv)
    x, w, lens, cache = si.make_decode_inputs(c, batch=3, capacity=70, len_lo=1, len_hi=69,
                                              gains="random")
    cfg = oracle_cfg(c)
    y_e, r_e = orc.mla_decode_expanded(cfg, w, x, cache, lens)
    y_a, r_a = orc.mla_decode_absorbed(cfg, w, x, cache, lens)
    np.testing.assert_array_equal(r_a, r_e)
    np.testing.assert_allclose(y_a, y_e, rtol=1e-12, atol=1e-15)


def test_decode_with_empty_cache_is_single_token_prefill():
    cfg, x, w = _tiny_inputs(S=1, B=2)
    cache = np.zeros((2, 4, cfg.kv_lora_rank + cfg.qk_rope_head_dim))
    y, _ = orc.mla_decode_absorbed(cfg, w, x[:, 0], cache, np.array([0, 0]))
    np.testing.assert_allclose(y, orc.mla_prefill(cfg, w, x)[:, 0], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_decode_after_prefill(conv):
    # decoding token S over the latent rows a prefill of tokens 0..S-1 wrote
    # equals row S of a prefill of tokens 0..S
    c = shrink(si.CONFIGS["small"], rope=conv)
    S = 40
    x, w = si.make_inputs(c, seq=S + 1, batch=2, gains="random")
    cfg = oracle_cfg(c)
    y_full = orc.mla_prefill(cfg, w, x)
    _, inter = orc.mla_prefill(cfg, w, x[:, :S], want_intermediates=True)
    cache = np.concatenate([inter["c_kv"], inter["k_pe"]], axis=-1)
    y_dec, new_rows = orc.mla_decode_absorbed(cfg, w, x[:, S], cache, np.array([S, S]))
    np.testing.assert_allclose(y_dec, y_full[:, S], rtol=1e-11, atol=1e-14)
    _, inter_full = orc.mla_prefill(cfg, w, x, want_intermediates=True)
    np.testing.assert_allclose(new_rows[:, :128], inter_full["c_kv"][:, S], rtol=1e-13)
    np.testing.assert_allclose(new_rows[:, 128:], inter_full["k_pe"][:, S], rtol=1e-12,
                               atol=1e-14)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_multi_token_decode_equals_sequential_decodes(conv):
    # T new tokens in one step equal T single-token decodes, each appending
    # its row before the next one runs
    c = shrink(si.CONFIGS["small"], rope=conv)
    T, B = 3, 3
    x1, w, lens, cache = si.make_decode_inputs(c, batch=B, capacity=80, len_lo=0, len_hi=70,
                                               gains="random")
    xs, _ = si.make_inputs(c, seq=T, batch=B, gains="random")
    cfg = oracle_cfg(c)
    y_m, rows_m = orc.mla_decode_absorbed_multi(cfg, w, xs, cache, lens)
    cache_s = cache.astype(np.float64).copy()
    for t in range(T):
        y_t, row_t = orc.mla_decode_absorbed(cfg, w, xs[:, t], cache_s, lens + t)
        for b in range(B):
            cache_s[b, lens[b] + t] = row_t[b]
        np.testing.assert_allclose(y_m[:, t], y_t, rtol=1e-12, atol=1e-15)
        np.testing.assert_array_equal(rows_m[:, t], row_t)


def test_multi_token_decode_equals_prefill_tail():
    # decoding tokens S..S+T-1 over a prefill's latent rows of tokens 0..S-1
    # equals rows S..S+T-1 of a prefill of all S+T tokens
    c = shrink(si.CONFIGS["small"], rope="interleaved")
    S, T = 30, 4
    x, w = si.make_inputs(c, seq=S + T, batch=2, gains="random")
    cfg = oracle_cfg(c)
    y_full = orc.mla_prefill(cfg, w, x)
    _, inter = orc.mla_prefill(cfg, w, x[:, :S], want_intermediates=True)
    cache = np.concatenate([inter["c_kv"], inter["k_pe"]], axis=-1)
    y_dec, _ = orc.mla_decode_absorbed_multi(cfg, w, x[:, S:], cache, np.array([S, S]))
    np.testing.assert_allclose(y_dec, y_full[:, S:], rtol=1e-11, atol=1e-14)


def test_latent_cache_is_small():
    # per token the cache holds c_kv (512) + k_pe (64) = 576 values, against
    # 2 * 128 heads * 128 = 32768 for per-head K and V at V3 sizes
    c = si.V3
    assert c["kv_lora_rank"] + c["qk_rope_head_dim"] == 576
    assert 576 / (2 * c["num_attention_heads"] * c["qk_nope_head_dim"]) < 0.02


# ------------------------------------------------------- optional c_kv norm --

def _with_kv_norm(w, rng, gain_one=False):
    w = dict(w)
    r = w["w_down_kv"].shape[0]
    w["kv_norm"] = np.ones(r) if gain_one else 1.0 + 0.1 * rng.standard_normal(r)
    return w


def test_kv_norm_latent_rows_have_unit_rms_and_match_torch():
    # with gains 1 and eps 0 every cached c_kv row has RMS 1; with random
    # gains it is torch's rms_norm of x W_dkv^T
    cfg, x, w = _tiny_inputs()
    rng = np.random.default_rng(41)
    cfg0 = orc.Cfg(**{**cfg.__dict__, "rms_norm_eps": 0.0})
    _, inter = orc.mla_prefill(cfg0, _with_kv_norm(w, rng, gain_one=True), x, want_intermediates=True)
    np.testing.assert_allclose(np.sqrt(np.mean(inter["c_kv"] ** 2, axis=-1)), 1.0, rtol=1e-12)
    wn = _with_kv_norm(w, rng)
    _, inter = orc.mla_prefill(cfg, wn, x, want_intermediates=True)
    ref = F.rms_norm(torch.from_numpy(x @ w["w_down_kv"].T), (w["w_down_kv"].shape[0],),
                     torch.from_numpy(wn["kv_norm"]), eps=cfg.rms_norm_eps).numpy()
    np.testing.assert_allclose(inter["c_kv"], ref, rtol=1e-12, atol=1e-14)


def test_kv_norm_makes_output_invariant_to_latent_scale():
    # the norm sits between w_down_kv and everything that reads c_kv (cache,
    # w_up_k, w_up_v): scaling w_down_kv leaves y unchanged at eps 0, and
    # without the norm it does not
    cfg, x, w = _tiny_inputs()
    cfg0 = orc.Cfg(**{**cfg.__dict__, "rms_norm_eps": 0.0})
    wn = _with_kv_norm(w, np.random.default_rng(42))
    ws = dict(wn, w_down_kv=wn["w_down_kv"] * 7.5)
    np.testing.assert_allclose(orc.mla_prefill(cfg0, ws, x), orc.mla_prefill(cfg0, wn, x),
                               rtol=1e-10, atol=1e-12)
    w_plain = {k: v for k, v in wn.items() if k != "kv_norm"}
    w_plain_s = dict(w_plain, w_down_kv=w_plain["w_down_kv"] * 7.5)
    assert np.abs(orc.mla_prefill(cfg0, w_plain_s, x) - orc.mla_prefill(cfg0, w_plain, x)).max() > 1e-3
    # an explicit None is the pages' reading (no norm)
    np.testing.assert_array_equal(orc.mla_prefill(cfg, dict(w, kv_norm=None), x),
                                  orc.mla_prefill(cfg, w, x))


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_kv_norm_decode_after_prefill_and_absorbed_equals_expanded(conv):
    # with the norm, the cached rows a prefill leaves serve the next decode
    # step, whose output is the prefill's next row; absorbed == expanded
    cfg, x, w = _tiny_inputs(conv, S=12)
    wn = _with_kv_norm(w, np.random.default_rng(43))
    full = orc.mla_prefill(cfg, wn, x)
    _, inter = orc.mla_prefill(cfg, wn, x[:, :11], want_intermediates=True)
    cache = np.concatenate([inter["c_kv"], inter["k_pe"]], axis=-1)
    cache = np.concatenate([cache, np.zeros((1, 4, cache.shape[-1]))], axis=1)
    lens = np.array([11])
    ya, rows = orc.mla_decode_absorbed(cfg, wn, x[:, 11], cache, lens)
    ye, _ = orc.mla_decode_expanded(cfg, wn, x[:, 11], cache, lens)
    np.testing.assert_allclose(ya, full[:, 11], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ya, ye, rtol=1e-12, atol=1e-13)
    _, inter12 = orc.mla_prefill(cfg, wn, x, want_intermediates=True)
    np.testing.assert_allclose(rows[0, :cfg.kv_lora_rank], inter12["c_kv"][0, 11], rtol=1e-12)
