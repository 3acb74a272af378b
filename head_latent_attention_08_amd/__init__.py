"""MI355X-native DeepSeek-V3 Multi-head Latent Attention forward.

The compute lives in libmla.so (hand-written gfx950 HIP kernels behind the C
ABI in include/mla.h); this package is its ctypes binding.
"""

from .mla import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    ROPE_HALF_SPLIT,
    ROPE_INTERLEAVED,
    MlaConfig,
    MlaError,
    RopeParams,
    load_library,
    mla_decode_absorbed,
    mla_decode_absorbed_multi,
    mla_decode_multi_workspace_size,
    mla_decode_layout_of,
    mla_decode_workspace_size,
    mla_attention_backward,
    mla_attention_backward_noalloc,
    mla_attention_backward_noalloc_max_rows,
    mla_fp8_gemm,
    mla_rmsnorm_backward,
    mla_fp8_quantize_blocks,
    mla_fp8_quantize_rows,
    mla_fp8_scale_pitch,
    mla_prefill_chunk,
    mla_prefill_chunk_workspace_size,
    mla_prefill_forward,
    mla_prefill_layout_of,
    mla_prefill_varlen_forward,
    mla_prefill_varlen_workspace_size,
    mla_prefill_workspace_size,
    mla_rope_apply,
    mla_set_stage_events,
    PREFILL_STAGES,
    DECODE_STAGES,
    mla_softmax_scale,
    mla_version,
)
