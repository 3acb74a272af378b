"""Seeded stress inputs shared by the GPU parity tests and the CPU tests that
derive their tolerances from the bf16 storage model (tests/bf16_emulation.py).
Shapes and draws only."""

from __future__ import annotations

import numpy as np

from tests.helpers import shrink, si


def sharp_logit_prefill(dtype="bf16", S=256):
    """The small config with the query weights x30 (seed 6000): logits of a
    few units, so the online softmax really rescales."""
    c = shrink(si.CONFIGS["small"], seed=6000, dtype=dtype)
    x, w = si.make_inputs(c, seq=S, gains="random", weight_scale={"w_up_q": 30.0, "w_qr": 30.0})
    return c, x, w


def decode_score_range(dtype):
    """Decode inputs whose cache rows after the first tile score far above
    it: w_up_k x40 and cache rows 100.. x8 (seed 6100)."""
    c = shrink(si.CONFIGS["small"], dtype=dtype)
    x, w, lens, cache = si.make_decode_inputs(c, batch=3, capacity=400, len_lo=200, len_hi=390,
                                              gains="random", seed=6100)
    w["w_up_k"] = si._store(w["w_up_k"] * 40.0, dtype)
    cache = cache.copy()
    cache[:, 100:] = si._store(cache[:, 100:] * 8.0, dtype)
    return c, x, w, lens, cache
