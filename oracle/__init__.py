"""Float64 CPU oracle for the DeepSeek-V3 Multi-head Latent Attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and the HIP library shares none with it.
"""

from .mla_oracle import (  # noqa: F401
    Cfg,
    rope_inv_freq,
    yarn_correction_range,
    yarn_inv_freq,
    yarn_mscale,
    cfg_inv_freq,
    cfg_cos_sin_scale,
    rope_cos_sin,
    rope_half_split,
    rope_interleaved,
    apply_rope,
    deinterleave_perm,
    rmsnorm,
    latent,
    softmax_scale,
    causal_attention,
    mla_prefill,
    mla_prefill_varlen,
    mla_prefill_rows,
    mla_decode_expanded,
    mla_decode_absorbed,
    mla_decode_absorbed_multi,
)
