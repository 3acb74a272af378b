"""The allocation-free attention backward (mla_attention_backward_noalloc)
against mla_attention_backward: two calls in a row, the second smaller, each
compared with the workspace entry point's output (same kernels: bitwise
equal) and with the float64 oracle; sizes beyond the built-in scratch are
rejected on the host."""

import numpy as np
import pytest
import torch

from oracle import attn_backward_oracle as ab
from tests.gpu_util import gpu, require_gpu, si
from tests.helpers import assert_close_rows

pytestmark = gpu


def _m():
    require_gpu()
    import head_latent_attention_08_amd as m
    return m


def _inputs(BH, S, dqk, dv, seed, dtype):
    bf = dtype == "bf16"
    q, k, v, do = si.make_attention_backward_inputs(BH, S, dqk, dv, seed, bf16=bf)
    scale = dqk ** -0.5
    o = ab.attention_forward_heads(q, k, v, scale)
    if bf:
        o = si.round_bf16(o.astype(np.float32)).astype(np.float64)
    td = torch.bfloat16 if bf else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(td).cuda()
    return (q, k, v, o, do, scale), tuple(dev(a) for a in (q, k, v, o, do))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_noalloc_matches_workspace_entry_point_twice(dtype):
    m = _m()
    # first call larger than the second, so stale scratch rows of the first
    # would show in the second if it read any row it had not written
    for BH, S, dqk, dv, seed in ((4, 300, 192, 128, 811), (2, 130, 64, 64, 812)):
        host, (q, k, v, o, do) = _inputs(BH, S, dqk, dv, seed, dtype)
        scale = host[-1]
        ref = m.mla_attention_backward(q, k, v, o, do, scale)
        dq = torch.full_like(q, float("nan"))
        dk = torch.full_like(k, float("nan"))
        dvv = torch.full_like(v, float("nan"))
        got = m.mla_attention_backward_noalloc(q, k, v, o, do, scale, dq=dq, dk=dk, dv=dvv)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), f"{name} differs from the workspace entry point ({BH}x{S})"
        qh, kh, vh, oh, doh, _ = host
        rq, rk, rv = ab.attention_backward_heads(qh, kh, vh, doh, scale, o=oh)
        for name, g, r in (("dq", got[0], rq), ("dk", got[1], rk), ("dv", got[2], rv)):
            g = g.float().cpu().numpy().reshape(-1, r.shape[-1]).astype(np.float64)
            r = r.reshape(-1, r.shape[-1])
            keep = np.abs(r).max(axis=1) > 1e-6 * np.abs(r).max()
            assert_close_rows(g[keep], r[keep], dtype, name)


def test_noalloc_rejects_more_rows_than_its_scratch():
    m = _m()
    mx = m.mla_attention_backward_noalloc_max_rows()
    assert mx == 1 << 21
    # a [BH, S] larger than the scratch is refused before any launch; the
    # tensors are never touched, so a tiny stand-in buffer suffices for the
    # pointers (the shape check is the library's, on sizes only)
    import ctypes
    lib = m.load_library()
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    st = lib.mla_attention_backward_noalloc(0, mx // 1024 + 1, 1024, 64, 64, 0.125, p, p, p, p, p, p, p, p,
                                            None)
    assert st == m.mla.MLA_ERR_INVALID_ARGUMENT
    assert b"scratch" in lib.mla_last_error()
