"""Helpers for GPU tests: device copies of the seeded inputs and configs."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth_inputs as si

gpu = pytest.mark.gpu


def have_gpu() -> bool:
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")


def mla_cfg(c: dict, rope=None, dtype=None, **over):
    import head_latent_attention_08_amd as m
    conv = rope or c["rope"]
    kw = dict(hidden_size=c["hidden_size"], num_heads=c["num_attention_heads"],
              q_lora_rank=c["q_lora_rank"], kv_lora_rank=c["kv_lora_rank"],
              qk_nope_head_dim=c["qk_nope_head_dim"], qk_rope_head_dim=c["qk_rope_head_dim"],
              v_head_dim=c["v_head_dim"], rms_norm_eps=1e-6, rope_theta=10000.0,
              rope_convention=m.ROPE_INTERLEAVED if conv == "interleaved" else m.ROPE_HALF_SPLIT,
              rope_factor=c.get("rope_factor", 1.0),
              original_max_position=c.get("original_max_position_embeddings", 4096),
              beta_fast=c.get("beta_fast", 32.0), beta_slow=c.get("beta_slow", 1.0),
              mscale=c.get("mscale", 1.0), mscale_all_dim=c.get("mscale_all_dim", 1.0),
              dtype=m.DTYPE_BF16 if (dtype or c["dtype"]) == "bf16" else m.DTYPE_F32)
    kw.update(over)
    return m.MlaConfig(**kw)


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device).contiguous()


def weights_to_dev(w: dict, dtype: str) -> dict:
    return {k: to_dev(v, dtype) for k, v in w.items()}


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ws_view(ws: torch.Tensor, offset: int, shape, dtype: torch.dtype, row_pitch=None):
    """A typed view of an intermediate inside the uint8 workspace."""
    es = torch.tensor([], dtype=dtype).element_size()
    n = int(np.prod(shape)) if row_pitch is None else shape[0] * row_pitch
    flat = ws[offset: offset + n * es].view(dtype)
    if row_pitch is None:
        return flat.view(*shape)
    return flat.view(shape[0], row_pitch)[:, : shape[1]]


__all__ = ["gpu", "have_gpu", "require_gpu", "mla_cfg", "to_dev", "weights_to_dev", "to_np",
           "ws_view", "si"]
