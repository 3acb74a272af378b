"""Shared test helpers: config conversion and the per-row error measure."""

from __future__ import annotations

import numpy as np

import synth_inputs as si
from oracle import Cfg


def oracle_cfg(c: dict, rope=None, **over) -> Cfg:
    """Oracle config from a synthetic-input config dict."""
    kw = dict(
        hidden_size=c["hidden_size"],
        num_attention_heads=c["num_attention_heads"],
        q_lora_rank=c["q_lora_rank"],
        kv_lora_rank=c["kv_lora_rank"],
        qk_nope_head_dim=c["qk_nope_head_dim"],
        qk_rope_head_dim=c["qk_rope_head_dim"],
        v_head_dim=c["v_head_dim"],
        rms_norm_eps=1e-6,
        rope_theta=10000.0,
        rope_convention=rope or c["rope"],
        rope_factor=c.get("rope_factor", 1.0),
        original_max_position_embeddings=c.get(
            "original_max_position_embeddings", 4096),
        beta_fast=c.get("beta_fast", 32.0),
        beta_slow=c.get("beta_slow", 1.0),
        mscale=c.get("mscale", 1.0),
        mscale_all_dim=c.get("mscale_all_dim", 1.0),
    )
    kw.update(over)
    return Cfg(**kw)


def shrink(c: dict, **over) -> dict:
    d = dict(c)
    d.update(over)
    return d


def row_errors(got, ref):
    """Per-token-row error measures over the last axis.

    rel_r = max_c |g - o| / max_c |o|; abs_r = max_c |g - o| / rms_c(o).
    Rows are judged separately because the output scale falls with the row
    index (later rows average more keys)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    o = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    d = np.abs(g - o).max(axis=1)
    mx = np.abs(o).max(axis=1)
    rms = np.sqrt(np.mean(o * o, axis=1))
    rel = d / np.maximum(mx, 1e-300)
    ab = d / np.maximum(rms, 1e-300)
    return rel, ab


def assert_close_rows(got, ref, dtype, what=""):
    """fp32: max_r rel_r <= 1e-4.  bf16: max_r rel_r <= 2e-2 and
    max_r abs_r <= 3e-2 (unit-scaled)."""
    rel, ab = row_errors(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite"
    if dtype == "fp32":
        assert rel.max() <= 1e-4, f"{what}: max rel {rel.max():.3e} (row {rel.argmax()})"
    else:
        assert rel.max() <= 2e-2, f"{what}: max rel {rel.max():.3e} (row {rel.argmax()})"
        assert ab.max() <= 3e-2, f"{what}: max abs {ab.max():.3e} (row {ab.argmax()})"
    return rel.max(), ab.max()


__all__ = ["oracle_cfg", "shrink", "row_errors", "assert_close_rows", "si"]
