"""GPU parity of the causal attention backward (dQ, dK, dV) against the
float64 oracle in oracle/attn_backward_oracle.py, element by element per row:
fp32 max per-row relative error <= 1e-4; bf16 <= 2e-2 relative and <= 3e-2
absolute on unit-scaled rows.  Also the RoPE backward: the transpose of a
rotation is the rotation by the negated angle, i.e. mla_rope_apply at the
negated positions."""

import numpy as np
import pytest
import torch

import oracle as orc
from oracle import attn_backward_oracle as ab
from tests.gpu_util import gpu, require_gpu, si
from tests.helpers import assert_close_rows

pytestmark = gpu


def _m():
    require_gpu()
    import head_latent_attention_08_amd as m
    return m


def _run(BH, S, dqk, dv, seed, dtype):
    m = _m()
    bf = dtype == "bf16"
    q, k, v, do = si.make_attention_backward_inputs(BH, S, dqk, dv, seed, bf16=bf)
    scale = dqk ** -0.5
    o = ab.attention_forward_heads(q, k, v, scale)
    td = torch.bfloat16 if bf else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(td).cuda()
    gq, gk, gv = m.mla_attention_backward(dev(q), dev(k), dev(v), dev(o), dev(do), scale)
    torch.cuda.synchronize()
    # the oracle takes the forward output as the kernel was handed it
    o_given = si.round_bf16(o.astype(np.float32)).astype(np.float64) if bf else o
    rq, rk, rv = ab.attention_backward_heads(q, k, v, do, scale, o=o_given)
    for name, g, r in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
        g = g.float().cpu().numpy().reshape(-1, r.shape[-1]).astype(np.float64)
        r = r.reshape(-1, r.shape[-1])
        # rows whose exact gradient vanishes (the first query of each head sees
        # only its own key) are checked against the tensor's scale instead
        # (a gradient scale from the inputs: |dout| |v| |q or k| d_v)
        top = float(np.abs(do).max() * np.abs(v).max() * max(np.abs(q).max(), np.abs(k).max()) * dv)
        zero = np.abs(r).max(axis=1) <= 1e-9 * top
        tol = 1e-5 if dtype == "fp32" else 1e-2
        assert np.all(np.abs(g[zero]) <= tol * top), f"{name}: vanishing rows not ~0"
        if np.any(~zero):
            assert_close_rows(g[~zero], r[~zero], dtype, name)


@pytest.mark.parametrize("BH,S,dqk,dv", [(3, 200, 40, 24), (2, 64, 16, 8), (1, 1, 8, 8), (2, 300, 192, 128)])
def test_backward_fp32_matches_oracle(BH, S, dqk, dv):
    _run(BH, S, dqk, dv, seed=BH * 1000 + S, dtype="fp32")


@pytest.mark.parametrize("BH,S,dqk,dv", [(2, 130, 64, 64), (2, 257, 192, 128)])
def test_backward_bf16_matches_oracle(BH, S, dqk, dv):
    _run(BH, S, dqk, dv, seed=BH * 1000 + S + 1, dtype="bf16")


def test_backward_bf16_v3_bench_shape_sampled_heads():
    # the bench launch: 128 heads x 4096 tokens, d_qk 192, d_v 128, bf16.
    # Heads are independent, so 8 of them (spread over the grid's XCD groups)
    # are checked in full against the oracle; the others carry o = 0.
    m = _m()
    BH, S, dqk, dv = 128, 4096, 192, 128
    print(f"attention backward bench shape: BH={BH} S={S} {dqk}/{dv} bf16, seed 9600", flush=True)
    q, k, v, do = si.make_attention_backward_inputs(BH, S, dqk, dv, 9600, bf16=True)
    scale = dqk ** -0.5
    heads = [0, 15, 16, 63, 64, 97, 112, 127]
    o = np.zeros((BH, S, dv), dtype=np.float32)
    o[heads] = si.round_bf16(ab.attention_forward_heads(q[heads], k[heads], v[heads], scale).astype(np.float32))
    dev = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()
    gq, gk, gv = m.mla_attention_backward(dev(q), dev(k), dev(v), dev(o), dev(do), scale)
    torch.cuda.synchronize()
    sel = torch.tensor(heads, device="cuda")
    got = [g[sel].float().cpu().numpy().astype(np.float64) for g in (gq, gk, gv)]
    for i, h in enumerate(heads):
        ref = ab.causal_attention_backward(q[h], k[h], v[h], do[h], scale, o[h])
        for name, g, r in zip(("dq", "dk", "dv"), (x[i] for x in got), ref):
            # the first query's gradient vanishes (it sees only its own key)
            top = float(np.abs(r).max())
            zero = np.abs(r).max(axis=1) <= 1e-9 * top
            assert np.all(np.abs(g[zero]) <= 1e-2 * top), f"head {h} {name}: vanishing rows not ~0"
            assert_close_rows(g[~zero], r[~zero], "bf16", f"head {h} {name}")


def test_backward_empty_launches_nothing():
    m = _m()
    z = torch.empty((0, 8, 8), device="cuda")
    dq, dk, dv = m.mla_attention_backward(z, z, z, z, z, 0.5)
    assert dq.numel() == 0


def test_rope_backward_is_rotation_by_negated_positions():
    # <R(p) x, y> = <x, R(-p) y>: the gradient of RoPE is RoPE at -p
    m = _m()
    rng = np.random.default_rng(41)
    n, h, d = 50, 3, 64
    y = rng.standard_normal((n, h, d)).astype(np.float32)
    pos = rng.integers(0, 30000, n).astype(np.int32)
    for conv, cflag in (("half_split", m.ROPE_HALF_SPLIT), ("interleaved", m.ROPE_INTERLEAVED)):
        cfg = orc.Cfg(64, h, 8, 8, 8, d, 8, rope_convention=conv)
        yd = torch.from_numpy(y.copy()).cuda()
        m.mla_rope_apply(yd, torch.from_numpy(-pos).cuda(), m.RopeParams(10000.0, cflag, 1.0, 4096, 32.0, 1.0, 1.0, 1.0))
        torch.cuda.synchronize()
        ref = orc.apply_rope(y.astype(np.float64), -pos.astype(np.int64), cfg)
        assert_close_rows(yd.cpu().numpy().reshape(n, -1), ref.reshape(n, -1), "fp32", "rope backward")
        x = rng.standard_normal((n, h, d))
        lhs = np.sum(orc.apply_rope(x, pos.astype(np.int64), cfg) * y)
        rhs = np.sum(x * ref)
        assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + 1)


@pytest.mark.parametrize("dtype,rows,n", [("fp32", 300, 1536), ("fp32", 7, 100), ("bf16", 257, 1536)])
def test_rmsnorm_backward_matches_oracle(dtype, rows, n):
    # the RMSNorm on c_q (r_q = 1536 at V3): dx per row, dg over all rows
    m = _m()
    bf = dtype == "bf16"
    rng = np.random.default_rng(rows + n)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    dy = rng.standard_normal((rows, n)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
    if bf:
        x, dy, g = si.round_bf16(x), si.round_bf16(dy), si.round_bf16(g)
    td = torch.bfloat16 if bf else torch.float32
    dev = lambda a: torch.from_numpy(a).to(td).cuda()
    dx, dg = m.mla_rmsnorm_backward(dev(x), dev(dy), dev(g), 1e-6)
    torch.cuda.synchronize()
    rdx, rdg = ab.rmsnorm_backward(x, g, dy, 1e-6)
    assert_close_rows(dx.float().cpu().numpy(), rdx, dtype, "dx")
    # dg sums rows of products rounded per step in fp32: relative to the
    # summed magnitudes
    mag = np.sum(np.abs(dy.astype(np.float64) * x), axis=0) / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1)).min()
    err = np.abs(dg.cpu().numpy() - rdg)
    assert np.all(err <= 1e-5 * mag + 1e-6), err.max()
