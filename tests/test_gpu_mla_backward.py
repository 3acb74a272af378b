"""GPU parity of the assembled MLA backward (mla_backward) against the
float64 chain-rule oracle (oracle/mla_backward_oracle.py): dx and every
weight's gradient, row by row (a weight gradient's rows are its output
features), on the tiny config in fp32 (1e-4), the small config in bf16 with
both RoPE conventions and with / without the norm on c_kv, ragged lengths,
YaRN, and the V3 dimensions (128 heads, hidden 7168) at a short sequence."""

import numpy as np
import pytest
import torch

from oracle.mla_backward_oracle import mla_backward as oracle_backward
from tests import bf16_emulation as be
from tests.gpu_util import gpu, mla_cfg, require_gpu, si, to_dev, to_np, weights_to_dev
from tests.helpers import oracle_cfg, row_errors, shrink

pytestmark = gpu


def _m():
    require_gpu()
    import head_latent_attention_08_amd as m
    return m


def _run(c, conv, S, B, seed, kv_norm=False, dy_scale=1.0):
    m = _m()
    dt = c["dtype"]
    x, w = si.make_inputs(c, seq=S, batch=B, gains="random", seed=seed)
    rng = np.random.default_rng(seed + 7)
    if kv_norm:
        w["kv_norm"] = si._store(1.0 + 0.2 * rng.standard_normal(c["kv_lora_rank"]).astype(np.float32), dt)
    dy = si._store(rng.standard_normal(x.shape).astype(np.float32) * np.float32(dy_scale), dt)
    cfg = mla_cfg(c, rope=conv)
    print(f"mla backward: {c['hidden_size']}/{c['num_attention_heads']} heads B={B} S={S} {dt} {conv} "
          f"kv_norm={kv_norm} seed {seed}", flush=True)
    dx, grads = m.mla_backward(cfg, weights_to_dev(w, dt), to_dev(x, dt), to_dev(dy, dt))
    torch.cuda.synchronize()
    ocfg = oracle_cfg(c, rope=conv)
    rdx, rg = oracle_backward(ocfg, w, x, dy)
    model = be.mla_backward_bf16(ocfg, w, x, dy) if dt == "bf16" else None
    return dt, dx, grads, rdx, rg, model


def _rows(a, like):
    return a.reshape(1, -1) if like.ndim == 1 else a.reshape(-1, like.shape[-1])


def _check(dt, got, ref, model, what, natural):
    """Row by row (a weight gradient's rows are its output features).  fp32:
    rel <= 1e-4.  bf16: bf16 storage of the chain's intermediates alone costs
    about the strict bound on gradients (the storage model of
    tests/bf16_emulation.mla_backward_bf16 reaches 2-3e-2 unit-scaled abs),
    so the bounds are max(strict, 1.6 x modelled) per tensor.  Rows whose
    exact gradient vanishes (e.g. every query gradient of one-token
    sequences: dS = P (dP - rowsum(dO O)) with P = 1) are checked against the
    gradients' natural scale (the largest of all of them) instead."""
    got, ref = _rows(got, ref), _rows(ref, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    zero = np.abs(ref).max(axis=1) <= 1e-9 * natural
    if np.any(zero):
        tol0 = 1e-5 if dt == "fp32" else 1e-2
        assert np.abs(got[zero]).max() <= tol0 * natural, f"{what}: vanishing rows not ~0"
    if not np.any(~zero):
        return
    rel, ab = row_errors(got[~zero], ref[~zero])
    if dt == "fp32":
        assert rel.max() <= 1e-4, f"{what}: max rel {rel.max():.3e}"
        return
    m_rel, m_ab = (e.max() for e in row_errors(_rows(model, model)[~zero], ref[~zero]))
    lim_rel, lim_ab = be.bound(2e-2, m_rel), be.bound(3e-2, m_ab)
    print(f"  {what}: rel {rel.max():.3e} abs {ab.max():.3e} (model {m_rel:.3e} / {m_ab:.3e})", flush=True)
    assert rel.max() <= lim_rel and ab.max() <= lim_ab, (what, rel.max(), ab.max(), lim_rel, lim_ab)


def _compare(dt, dx, grads, rdx, rg, model):
    mdx, mg = model if model is not None else (None, {})
    natural = max([np.abs(rdx).max()] + [np.abs(r).max() for r in rg.values()])
    _check(dt, to_np(dx), rdx, mdx, "dx", natural)
    assert set(grads) == set(rg)
    for name, ref in rg.items():
        _check(dt, to_np(grads[name]), ref, mg.get(name), name, natural)


@pytest.mark.parametrize("conv", ["half_split", "interleaved"])
def test_mla_backward_tiny_fp32(conv):
    c = si.CONFIGS["tiny"]
    _compare(*_run(c, conv, S=16, B=2, seed=1300))


def test_mla_backward_tiny_fp32_kv_norm_yarn():
    c = shrink(si.CONFIGS["tiny"], rope_factor=8.0, original_max_position_embeddings=4, beta_fast=2.0,
               beta_slow=1.0, mscale=0.9, mscale_all_dim=1.1)
    _compare(*_run(c, "interleaved", S=24, B=1, seed=1301, kv_norm=True))


@pytest.mark.parametrize("conv,kv_norm", [("interleaved", False), ("half_split", True)])
def test_mla_backward_small_bf16(conv, kv_norm):
    c = si.CONFIGS["small"]
    _compare(*_run(c, conv, S=130, B=2, seed=1302 + kv_norm, kv_norm=kv_norm))


def test_mla_backward_small_bf16_large_tile_products():
    # 512 tokens: every weight-gradient product with 512+ output rows and the
    # dc / dx products run on the large-tile kernel, their transposed
    # operands rewritten K-contiguous first
    c = si.CONFIGS["small"]
    _compare(*_run(c, "half_split", S=256, B=2, seed=1307, kv_norm=True))


def test_mla_backward_small_fp32_ragged():
    # 1 and 67 tokens: partial tiles everywhere, one-token sequences
    c = shrink(si.CONFIGS["small"], dtype="fp32")
    _compare(*_run(c, "interleaved", S=67, B=1, seed=1304))
    _compare(*_run(c, "half_split", S=1, B=3, seed=1305))


def test_mla_backward_v3_dims():
    c = si.CONFIGS["v3_prefill"]
    _compare(*_run(c, "interleaved", S=96, B=1, seed=1306))
