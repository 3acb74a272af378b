"""GPU parity at DeepSeek-V3 sizes, in the launch configuration the bench
times: the full forward runs on the GPU and the oracle recomputes sampled
output rows (prefill) or whole sequences (decode) one by one in float64.
Also bitwise causality, bitwise run-to-run determinism, decode after prefill
and the RoPE convention equivalence on the full forward."""

import numpy as np
import pytest
import torch

import oracle as orc
from tests.gpu_util import gpu, mla_cfg, require_gpu, si, to_dev, to_np, weights_to_dev
from tests.helpers import assert_close_rows, oracle_cfg, shrink

pytestmark = gpu


def _m():
    require_gpu()
    import head_latent_attention_08_amd as m
    return m


def _prefill(c, conv, x, w, dtype="bf16"):
    m = _m()
    cfg = mla_cfg(c, rope=conv)
    y, lat, ws = m.mla_prefill_forward(cfg, weights_to_dev(w, dtype), to_dev(x, dtype),
                                       want_latent=True)
    torch.cuda.synchronize()
    return y, lat


def test_v3_prefill_sampled_rows():
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c)
    print("v3 prefill: B=1 S=4096 interleaved, seed 3000", flush=True)
    y, lat = _prefill(c, "interleaved", x, w)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 2047, 4095],
                                     np.random.default_rng(3001).choice(4096, 24, replace=False)]))
    ref, ref_lat = orc.mla_prefill_rows(oracle_cfg(c), w, x, rows)
    assert_close_rows(to_np(y[0, rows]), ref, "bf16", "y rows")
    assert_close_rows(to_np(lat[0]), ref_lat, "bf16", "latent rows")


def test_v3_prefill_varlen_sampled_rows():
    # three V3 sequences packed into 4096 tokens; sampled rows of each against
    # the oracle's prefill of that sequence alone
    m = _m()
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c)
    lens = [1000, 2500, 596]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    print(f"v3 varlen: lens {lens}, seed 3000", flush=True)
    cfg = mla_cfg(c, rope="interleaved")
    y, lat, _ = m.mla_prefill_varlen_forward(cfg, weights_to_dev(w, "bf16"), to_dev(x[0], "bf16"),
                                             torch.from_numpy(cu).cuda(), want_latent=True)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        a = int(cu[b])
        rows = np.unique(np.array([0, 1, 31, 32, L // 2, L - 1]))
        ref, ref_lat = orc.mla_prefill_rows(oracle_cfg(c), w, x[:, a:a + L], rows)
        assert_close_rows(to_np(y[a + rows]), ref, "bf16", f"seq {b} y rows")
        assert_close_rows(to_np(lat[a:a + L]), ref_lat, "bf16", f"seq {b} latent")


def test_v3_prefill_chunk_after_prefill_sampled_rows():
    # V3: prefill 3000 tokens into the latent cache, then the remaining 1096
    # as one expanded chunk; sampled chunk rows against the oracle's prefill
    # of all 4096 tokens
    m = _m()
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c)
    L, T = 3000, 1096
    print(f"v3 chunk: prefix {L}, chunk {T}, seed 3000", flush=True)
    cfg = mla_cfg(c, rope="interleaved")
    wd = weights_to_dev(w, "bf16")
    _, lat, _ = m.mla_prefill_forward(cfg, wd, to_dev(x[:, :L], "bf16"), want_latent=True)
    cache = torch.zeros((1, L + T, lat.shape[-1]), dtype=torch.bfloat16, device="cuda")
    cache[0, :L] = lat[0]
    y, _ = m.mla_prefill_chunk(cfg, wd, to_dev(x[:, L:], "bf16"), cache,
                               torch.tensor([L], dtype=torch.int32, device="cuda"), L + T)
    torch.cuda.synchronize()
    rows = np.array([L, L + 1, L + 31, L + 32, L + 547, L + T - 1])
    ref, _ = orc.mla_prefill_rows(oracle_cfg(c), w, x, rows)
    assert_close_rows(to_np(y[0, rows - L]), ref, "bf16", "chunk rows")


def test_v3_prefill_half_split_spot_check():
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c, seq=1024)
    y, lat = _prefill(c, "half_split", x, w)
    rows = np.array([0, 5, 511, 1000, 1023])
    ref, _ = orc.mla_prefill_rows(oracle_cfg(c, rope="half_split"), w, x, rows)
    assert_close_rows(to_np(y[0, rows]), ref, "bf16", "y rows")


@pytest.mark.timeout(400)
def test_v3_yarn_long_context_sampled_rows():
    c = si.CONFIGS["v3_yarn"]
    x, w = si.make_inputs(c)
    print("v3 yarn: B=1 S=32768 interleaved factor 40, seed 5000", flush=True)
    y, lat = _prefill(c, "interleaved", x, w)
    rows = si.sample_rows(c, 32768)
    yr = to_np(y[0, torch.from_numpy(rows).cuda()])
    del y
    print(f"v3 yarn: oracle on {len(rows)} rows", flush=True)
    ref, ref_lat = orc.mla_prefill_rows(oracle_cfg(c), w, x, rows)
    assert_close_rows(yr, ref, "bf16", "y rows")
    assert_close_rows(to_np(lat[0]), ref_lat, "bf16", "latent rows")


def test_p5_shape_conventions():
    # the shape the RoPE convention thread compares at: seq 2048, 128 heads,
    # rope dim 64 (other sizes V3).  Each convention matches the oracle, the
    # two differ on the same weights, and agree once w_qr / w_kr rows are
    # permuted by the even/odd de-interleave.
    c = shrink(si.CONFIGS["v3_prefill"], seed=7000)
    x, w = si.make_inputs(c, seq=2048)
    rows = np.array([0, 1, 100, 1024, 2047])
    y_il, _ = _prefill(c, "interleaved", x, w)
    y_hs, _ = _prefill(c, "half_split", x, w)
    P = orc.deinterleave_perm(64)
    w2 = dict(w)
    w2["w_qr"] = w["w_qr"].reshape(128, 64, -1)[:, P].reshape(128 * 64, -1)
    w2["w_kr"] = w["w_kr"][P]
    y_hs_perm, _ = _prefill(c, "half_split", x, w2)
    refs = {}
    for conv, y in (("interleaved", y_il), ("half_split", y_hs)):
        refs[conv], _ = orc.mla_prefill_rows(oracle_cfg(c, rope=conv), w, x, rows)
        assert_close_rows(to_np(y[0, rows]), refs[conv], "bf16", conv)
    yi, yh, yp = to_np(y_il[0]), to_np(y_hs[0]), to_np(y_hs_perm[0])
    assert_close_rows(yp, yi, "bf16", "permuted half-split vs interleaved")
    # with V3-scale weights the logits are nearly uniform, so the two
    # conventions differ only slightly; the GPU must reproduce the oracle's
    # difference itself, well above its own rounding
    d_ref = refs["half_split"][1:] - refs["interleaved"][1:]
    d_gpu = yh[rows[1:]] - yi[rows[1:]]
    assert np.corrcoef(d_ref.ravel(), d_gpu.ravel())[0, 1] > 0.95
    assert np.abs(d_ref).max() > 10 * np.abs(yp[rows[1:]] - yi[rows[1:]]).mean()


def test_q_rope_in_up_projection_sampled_rows():
    # At this shape (seq 2048, V3 sizes, bf16) the q up-projection rotates
    # q_pe in its epilogue from the table the k_pe rotation writes: the
    # workspace's q of sampled tokens (every head) against the oracle's
    # c_q -> RMSNorm -> up-projections -> RoPE at those positions, both
    # conventions.
    m = _m()
    c = shrink(si.CONFIGS["v3_prefill"], seed=7100)
    x, w = si.make_inputs(c, seq=2048)
    H, dn, dr = c["num_attention_heads"], c["qk_nope_head_dim"], c["qk_rope_head_dim"]
    rows = np.array([0, 1, 31, 255, 256, 1000, 2047])
    xs = np.asarray(x, dtype=np.float64)[0, rows]
    for conv in ("interleaved", "half_split"):
        print(f"q rows: seq 2048 {conv}, seed 7100", flush=True)
        cfg = mla_cfg(c, rope=conv)
        _, _, ws = m.mla_prefill_forward(cfg, weights_to_dev(w, "bf16"), to_dev(x, "bf16"))
        torch.cuda.synchronize()
        lay = m.mla_prefill_layout_of(cfg, 1, 2048)
        q = to_np(ws[lay.q: lay.q + H * 2048 * (dn + dr) * 2].view(torch.bfloat16).view(H, 2048, dn + dr))
        oc = oracle_cfg(c, rope=conv)
        c_qn = orc.rmsnorm(xs @ np.asarray(w["w_down_q"], np.float64).T,
                           np.asarray(w["q_norm"], np.float64), oc.rms_norm_eps)
        q_nope = (c_qn @ np.asarray(w["w_up_q"], np.float64).T).reshape(len(rows), H, dn)
        q_pe = orc.apply_rope((c_qn @ np.asarray(w["w_qr"], np.float64).T).reshape(len(rows), H, dr), rows, oc)
        got = q[:, rows].transpose(1, 0, 2)  # [rows, H, dn + dr]
        assert_close_rows(got[..., dn:], q_pe, "bf16", f"q_pe {conv}")
        assert_close_rows(got[..., :dn], q_nope, "bf16", f"q_nope {conv}")


def test_causality_bitwise():
    # perturbing tokens t >= t0 leaves every output row t < t0 bit-identical
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=512)
    y0, _ = _prefill(c, "interleaved", x, w)
    x2 = x.copy()
    x2[:, 300:] = si.round_bf16(np.random.default_rng(9).standard_normal(x2[:, 300:].shape) * 3)
    y1, _ = _prefill(c, "interleaved", x2, w)
    assert torch.equal(y0[:, :300], y1[:, :300])
    assert not torch.equal(y0[:, 300:], y1[:, 300:])


def test_determinism_bitwise():
    m = _m()
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c)
    y0, l0 = _prefill(c, "interleaved", x, w)
    y1, l1 = _prefill(c, "interleaved", x, w)
    assert torch.equal(y0, y1) and torch.equal(l0, l1)
    xd, wd, lens, cache = si.make_decode_inputs(c, batch=9, capacity=700, len_lo=0, len_hi=690)
    cfg = mla_cfg(c)
    outs = []
    for _ in range(2):
        cache_d = to_dev(cache, "bf16")
        y, _ = m.mla_decode_absorbed(cfg, weights_to_dev(wd, "bf16"), to_dev(xd, "bf16"), cache_d,
                                     torch.from_numpy(lens).cuda())
        outs.append((y, cache_d))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.timeout(300)
def test_v3_determinism_bitwise():
    # At full size (many key tiles per query block, big-tile projections,
    # decode rows cut into ranges) every run gives bit-identical results,
    # whatever the workspace held before: no copy is read before it lands.
    m = _m()
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c)
    print("v3 determinism: prefill B=1 S=4096 x3, seed 3000", flush=True)
    cfg = mla_cfg(c)
    wd, xd = weights_to_dev(w, "bf16"), to_dev(x, "bf16")
    ws = torch.empty(m.mla_prefill_workspace_size(cfg, 1, x.shape[1]), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for fill in (0, 255, 0):
        ws.fill_(fill)
        y, lat, _ = m.mla_prefill_forward(cfg, wd, xd, workspace=ws, want_latent=True)
        torch.cuda.synchronize()
        outs.append((y, lat))
    for y, lat in outs[1:]:
        assert torch.equal(lat, outs[0][1])
        assert torch.equal(y, outs[0][0]), f"{(y != outs[0][0]).sum().item()} elements differ"
    del outs, ws, wd, xd
    c = si.CONFIGS["v3_decode"]
    print("v3 determinism: decode B=64 cap=8193 x2, seed 4000", flush=True)
    x, w, lens, cache = si.make_decode_inputs(c)
    cfg = mla_cfg(c)
    wd, xd, lens_d = weights_to_dev(w, "bf16"), to_dev(x, "bf16"), torch.from_numpy(lens).cuda()
    res = []
    for _ in range(2):
        cache_d = to_dev(cache, "bf16")
        y, _ = m.mla_decode_absorbed(cfg, wd, xd, cache_d, lens_d)
        torch.cuda.synchronize()
        res.append((y, cache_d))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


@pytest.mark.parametrize("name", ["small", "v3_prefill"])
def test_decode_after_prefill(name):
    # decoding token S over the latent rows a GPU prefill of tokens 0..S-1
    # wrote matches row S of the oracle prefill of tokens 0..S
    m = _m()
    c = si.CONFIGS[name]
    S, B = (200, 3) if name == "small" else (600, 2)
    x, w = si.make_inputs(c, seq=S + 1, batch=B, gains="random")
    cfg = mla_cfg(c, rope="interleaved")
    wd = weights_to_dev(w, "bf16")
    _, lat, _ = m.mla_prefill_forward(cfg, wd, to_dev(x[:, :S], "bf16"), want_latent=True)
    cap = S + 5
    cache = torch.zeros((B, cap, lat.shape[-1]), dtype=torch.bfloat16, device="cuda")
    cache[:, :S] = lat
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    y, _ = m.mla_decode_absorbed(cfg, wd, to_dev(x[:, S], "bf16"), cache, lens)
    torch.cuda.synchronize()
    ocfg = oracle_cfg(c, rope="interleaved")
    for b in range(B):
        ref, _ = orc.mla_prefill_rows(ocfg, w, x, [S], batch=b)
        assert_close_rows(to_np(y[b:b + 1]), ref, "bf16", f"seq {b}")


def test_v3_decode_full():
    m = _m()
    c = si.CONFIGS["v3_decode"]
    print("v3 decode: B=64 cap=8193 lens U{1024..8192}, seed 4000", flush=True)
    x, w, lens, cache = si.make_decode_inputs(c)
    cfg = mla_cfg(c)
    cache_d = to_dev(cache, "bf16")
    y, _ = m.mla_decode_absorbed(cfg, weights_to_dev(w, "bf16"), to_dev(x, "bf16"), cache_d,
                                 torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    ref, new_rows = orc.mla_decode_absorbed(oracle_cfg(c), w, x, cache, lens)
    assert_close_rows(to_np(y), ref, "bf16", "y")
    idx = torch.from_numpy(lens.astype(np.int64)).cuda()
    got_rows = to_np(cache_d[torch.arange(64, device="cuda"), idx])
    assert_close_rows(got_rows, new_rows, "bf16", "new cache rows")


def test_v3_decode_batch_4096_sampled():
    # the largest batch the decode entry takes, with short histories (0..40
    # rows): each row range holds many sequences; sampled sequences (and the
    # ends of the batch) against the oracle, with their new cache rows
    m = _m()
    c = si.CONFIGS["v3_decode"]
    B, cap = 4096, 41
    print(f"v3 decode: B={B} cap={cap} lens U{{0..40}}, seed 4200", flush=True)
    x, w, lens, cache = si.make_decode_inputs(c, batch=B, capacity=cap, len_lo=0, len_hi=40, seed=4200)
    cfg = mla_cfg(c)
    cache_d = to_dev(cache, "bf16")
    y, _ = m.mla_decode_absorbed(cfg, weights_to_dev(w, "bf16"), to_dev(x, "bf16"), cache_d,
                                 torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(4201)
    pick = np.unique(np.concatenate([[0, 1, 2494, 2495, 2496, B - 1], rng.choice(B, 40, replace=False)]))
    ref, new_rows = orc.mla_decode_absorbed(oracle_cfg(c), w, x[pick], cache[pick], lens[pick])
    assert_close_rows(to_np(y)[pick], ref, "bf16", "y")
    sel = torch.from_numpy(pick).cuda()
    got_rows = to_np(cache_d[sel, torch.from_numpy(lens[pick].astype(np.int64)).cuda()])
    assert_close_rows(got_rows, new_rows, "bf16", "new cache rows")


def test_v3_decode_expanded_spot_check():
    # the expanded definition (per-head K/V up-projection of every cached
    # row) on a few sequences agrees with the GPU's absorbed result
    m = _m()
    c = si.CONFIGS["v3_decode"]
    x, w, lens, cache = si.make_decode_inputs(c, batch=4, capacity=2100, len_lo=1024,
                                              len_hi=2099, seed=4100)
    cfg = mla_cfg(c)
    y, _ = m.mla_decode_absorbed(cfg, weights_to_dev(w, "bf16"), to_dev(x, "bf16"),
                                 to_dev(cache, "bf16"), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    ref, _ = orc.mla_decode_expanded(oracle_cfg(c), w, x, cache, lens)
    assert_close_rows(to_np(y), ref, "bf16", "y")


def test_v3_multi_token_decode():
    # two new tokens per sequence at V3 shapes (the verification pass of
    # speculative decoding): 16 sequences, lengths U{1024..4096}
    m = _m()
    c = si.CONFIGS["v3_decode"]
    B, T, cap = 16, 2, 4100
    print("v3 multi-token decode: B=16 T=2 cap=4100, seed 4200", flush=True)
    _, w, lens, cache = si.make_decode_inputs(c, batch=B, capacity=cap, len_lo=1024, len_hi=4096,
                                              seed=4200)
    xs, _ = si.make_inputs(c, seq=T, batch=B, seed=4200)
    cfg = mla_cfg(c)
    cache_d = to_dev(cache, "bf16")
    y, _ = m.mla_decode_absorbed_multi(cfg, weights_to_dev(w, "bf16"), to_dev(xs, "bf16"),
                                       cache_d, torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    ref, new_rows = orc.mla_decode_absorbed_multi(oracle_cfg(c), w, xs, cache, lens)
    yn = to_np(y)
    for t in range(T):
        assert_close_rows(yn[:, t], ref[:, t], "bf16", f"y token {t}")
    got = to_np(cache_d)
    for t in range(T):
        rows = np.stack([got[b, lens[b] + t] for b in range(B)])
        assert_close_rows(rows, new_rows[:, t], "bf16", f"new cache row {t}")
