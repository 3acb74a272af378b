"""The bf16 storage model behind the widened GPU tolerances (no GPU).

Two GPU parity inputs cannot meet the plain bf16 bound (rel 2e-2, abs 3e-2
unit-scaled): the sharp-logit prefill and the decode whose scores outrun the
first tile.  On both, bf16 storage of the intermediates alone (the model in
tests/bf16_emulation.py, exact arithmetic otherwise) already exceeds it, so
the GPU tests take max(strict, 1.6 x modelled) instead.  These tests pin the
model to the oracle (without rounding it is the oracle) and record that the
strict bound is out of reach on those inputs while ordinary inputs meet it.
"""

import numpy as np

import oracle as orc
from tests import bf16_emulation as be
from tests import stress_cases as sc
from tests.helpers import oracle_cfg, row_errors, si


def test_model_without_rounding_is_the_oracle():
    c, x, w = sc.sharp_logit_prefill(S=64)
    cfg = oracle_cfg(c, rope="half_split")
    np.testing.assert_allclose(be.prefill_bf16(cfg, w, x, rounding=False), orc.mla_prefill(cfg, w, x),
                               rtol=1e-12, atol=1e-12)
    c, x, w, lens, cache = sc.decode_score_range("bf16")
    cfg = oracle_cfg(c)
    np.testing.assert_allclose(be.decode_absorbed_bf16(cfg, w, x, cache, lens, rounding=False),
                               orc.mla_decode_absorbed(cfg, w, x, cache, lens)[0],
                               rtol=1e-12, atol=1e-12)


def test_ordinary_input_meets_strict_bound_under_the_model():
    # the small bf16 config: bf16 storage costs well under the strict bound
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=256, gains="random")
    cfg = oracle_cfg(c, rope="interleaved")
    rel, ab = row_errors(be.prefill_bf16(cfg, w, x), orc.mla_prefill(cfg, w, x))
    assert rel.max() < 2e-2 and ab.max() < 3e-2, (rel.max(), ab.max())


def test_sharp_logits_exceed_strict_bound_under_the_model():
    c, x, w = sc.sharp_logit_prefill()
    cfg = oracle_cfg(c, rope="half_split")
    rel, ab = row_errors(be.prefill_bf16(cfg, w, x), orc.mla_prefill(cfg, w, x))
    # abs: ~5.1e-2, beyond 3e-2 for any pipeline that stores q and k in bf16
    assert ab.max() > 3e-2, ab.max()
    assert be.bound(3e-2, ab.max()) < 1e-1


def test_decode_score_range_exceeds_strict_bound_under_the_model():
    c, x, w, lens, cache = sc.decode_score_range("bf16")
    cfg = oracle_cfg(c)
    rel, ab = row_errors(be.decode_absorbed_bf16(cfg, w, x, cache, lens),
                         orc.mla_decode_absorbed(cfg, w, x, cache, lens)[0])
    assert ab.max() > 3e-2, ab.max()
    assert be.bound(2e-2, rel.max()) < 3e-2 and be.bound(3e-2, ab.max()) < 1e-1


def test_backward_model_without_rounding_is_the_oracle():
    from oracle.mla_backward_oracle import mla_backward
    c = si.CONFIGS["small"]
    x, w = si.make_inputs(c, seq=20, batch=2, gains="random")
    dy = np.random.default_rng(5).standard_normal(x.shape)
    cfg = oracle_cfg(c, rope="interleaved")
    rdx, rg = mla_backward(cfg, w, x, dy)
    mdx, mg = be.mla_backward_bf16(cfg, w, x, dy, rounding=False)
    np.testing.assert_allclose(mdx, rdx, rtol=1e-12, atol=1e-12)
    for k in rg:
        np.testing.assert_allclose(mg[k], rg[k], rtol=1e-12, atol=1e-12, err_msg=k)
    # with bf16 storage the weight gradients move by about the strict bound
    mdx, mg = be.mla_backward_bf16(cfg, w, x, dy)
    _, ab = row_errors(mg["w_up_q"], rg["w_up_q"])
    assert 3e-3 < ab.max() < 1e-1, ab.max()
