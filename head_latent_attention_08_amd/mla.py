"""ctypes binding of libmla.so: argument marshalling only.

Every step of the forward runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  There is no fallback: if the
library is not built, or no GPU is present, the calls raise.

Names match the C ABI in include/mla.h.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime the library links against)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4

DTYPE_F32 = 0
DTYPE_BF16 = 1
ROPE_HALF_SPLIT = 0
ROPE_INTERLEAVED = 1

_TORCH_DTYPE = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mla status {status}: {message}")
        self.status = status
        self.message = message


class RopeParams(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_float), ("convention", ctypes.c_int32),
                ("factor", ctypes.c_float), ("original_max_position", ctypes.c_int32),
                ("beta_fast", ctypes.c_float), ("beta_slow", ctypes.c_float),
                ("mscale", ctypes.c_float), ("mscale_all_dim", ctypes.c_float)]


class Config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("q_lora_rank", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("rms_norm_eps", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("rope", RopeParams),
                ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_down_q", "q_norm", "w_up_q", "w_qr", "w_down_kv", "kv_norm", "w_kr", "w_up_k", "w_up_v",
        "wo")]


class Fp8Matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld", ctypes.c_int64), ("scales", ctypes.c_void_p),
                ("ld_scales", ctypes.c_int64)]


class Fp8Weights(ctypes.Structure):
    _fields_ = [(n, Fp8Matrix) for n in ("down", "q_up", "kv_up", "out")]


class WeightGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_down_q", "q_norm", "w_up_q", "w_qr", "w_down_kv", "kv_norm", "w_kr", "w_up_k", "w_up_v", "wo")]


class PrefillLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("c_q", "c_kv", "k_pe", "q", "k_nope", "v", "o")] + [
        ("ld_down", ctypes.c_int64), ("q_rms_part", ctypes.c_size_t), ("q_rms_chunks", ctypes.c_int64),
        ("total", ctypes.c_size_t)]


class DecodeLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("c_q", "c_kv", "q", "q_lat", "o_lat", "o")] + [
        ("ld_down", ctypes.c_int64), ("n_splits", ctypes.c_int64), ("split_len", ctypes.c_int64),
        ("total", ctypes.c_size_t)]


WEIGHT_NAMES = [f[0] for f in Weights._fields_]
# optional weights: absent or None means NULL (kv_norm: no norm on c_kv)
OPTIONAL_WEIGHTS = ("kv_norm",)

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m head_latent_attention_08_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    st = ctypes.c_int
    lib.mla_prefill_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64,
                                               ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_layout_of.argtypes = [ctypes.POINTER(Config), i64, i64,
                                          ctypes.POINTER(PrefillLayout)]
    lib.mla_prefill_forward.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P, i64,
                                        i64, P, P, P, ctypes.c_size_t, P]
    lib.mla_prefill_varlen_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_varlen_forward.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P,
                                               P, i64, i64, P, P, P, ctypes.c_size_t, P]
    lib.mla_prefill_chunk_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64, i64, i64,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_chunk.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P, i64, i64,
                                      P, i64, P, i64, P, P, ctypes.c_size_t, P]
    lib.mla_decode_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_layout_of.argtypes = [ctypes.POINTER(Config), i64, i64,
                                         ctypes.POINTER(DecodeLayout)]
    lib.mla_decode_absorbed.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P, i64,
                                        P, i64, P, P, P, ctypes.c_size_t, P]
    lib.mla_decode_multi_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64, i64,
                                                    ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_absorbed_multi.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P,
                                              i64, i64, P, i64, P, P, P, ctypes.c_size_t, P]
    lib.mla_rope_apply.argtypes = [P, ctypes.c_int32, i64, ctypes.c_int32, ctypes.c_int32, i64,
                                   i64, P, ctypes.POINTER(RopeParams), P]
    lib.mla_attention_backward_workspace_size.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_attention_backward.argtypes = [ctypes.c_int32, i64, i64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    for fn in ("mla_attention_backward_workspace_size", "mla_attention_backward"):
        getattr(lib, fn).restype = st
    lib.mla_attention_backward_noalloc.argtypes = [ctypes.c_int32, i64, i64, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_float, P, P, P, P, P, P, P, P, P]
    lib.mla_attention_backward_noalloc.restype = st
    lib.mla_attention_backward_noalloc_max_rows.argtypes = []
    lib.mla_attention_backward_noalloc_max_rows.restype = i64
    lib.mla_rmsnorm_backward.argtypes = [ctypes.c_int32, P, P, P, i64, ctypes.c_int32, ctypes.c_float, P, P,
                                         P, ctypes.c_size_t, P]
    lib.mla_rmsnorm_backward.restype = st
    lib.mla_rmsnorm_backward_workspace_size.argtypes = [i64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_rmsnorm_backward_workspace_size.restype = st
    lib.mla_backward_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_backward.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P, i64, i64, P, P,
                                 ctypes.POINTER(WeightGrads), P, ctypes.c_size_t, P]
    lib.mla_backward_workspace_size.restype = st
    lib.mla_backward.restype = st
    lib.mla_fp8_weights_size.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_fp8_prepare_weights.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), P, ctypes.c_size_t,
                                            ctypes.POINTER(Fp8Weights), P]
    lib.mla_prefill_fp8_workspace_size.argtypes = [ctypes.POINTER(Config), i64, i64,
                                                   ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_forward_fp8.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                                            ctypes.POINTER(Fp8Weights), P, i64, i64, P, P, P, ctypes.c_size_t, P]
    for fn in ("mla_fp8_weights_size", "mla_fp8_prepare_weights", "mla_prefill_fp8_workspace_size",
               "mla_prefill_forward_fp8"):
        getattr(lib, fn).restype = st
    lib.mla_fp8_scale_pitch.argtypes = [i64]
    lib.mla_fp8_scale_pitch.restype = i64
    lib.mla_fp8_quantize_rows.argtypes = [P, ctypes.c_int32, i64, i64, i64, P, i64, P, i64, P]
    lib.mla_fp8_quantize_blocks.argtypes = [P, ctypes.c_int32, i64, i64, i64, P, i64, P, i64, P]
    lib.mla_fp8_gemm.argtypes = [P, i64, P, i64, P, i64, P, i64, P, ctypes.c_int32, i64, i64, i64, i64, P]
    for fn in ("mla_fp8_quantize_rows", "mla_fp8_quantize_blocks", "mla_fp8_gemm"):
        getattr(lib, fn).restype = st
    for fn in ("mla_prefill_workspace_size", "mla_prefill_layout_of", "mla_prefill_forward",
               "mla_prefill_varlen_workspace_size", "mla_prefill_varlen_forward",
               "mla_prefill_chunk_workspace_size", "mla_prefill_chunk",
               "mla_decode_workspace_size", "mla_decode_layout_of", "mla_decode_absorbed",
               "mla_decode_multi_workspace_size", "mla_decode_absorbed_multi", "mla_rope_apply"):
        getattr(lib, fn).restype = st
    lib.mla_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
    lib.mla_set_stage_events.restype = st
    lib.mla_softmax_scale.argtypes = [ctypes.POINTER(Config)]
    lib.mla_softmax_scale.restype = ctypes.c_float
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, load_library().mla_last_error().decode())


@dataclass
class MlaConfig:
    """Python mirror of mla_config (DeepSeek-V3 field names)."""

    hidden_size: int
    num_heads: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    rms_norm_eps: float = 1e-6
    softmax_scale: float = 0.0
    rope_theta: float = 10000.0
    rope_convention: int = ROPE_HALF_SPLIT
    rope_factor: float = 1.0
    original_max_position: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 1.0
    dtype: int = DTYPE_BF16

    def rope_params(self) -> RopeParams:
        return RopeParams(self.rope_theta, self.rope_convention, self.rope_factor,
                          self.original_max_position, self.beta_fast, self.beta_slow,
                          self.mscale, self.mscale_all_dim)

    def c(self) -> Config:
        return Config(self.hidden_size, self.num_heads, self.q_lora_rank, self.kv_lora_rank,
                      self.qk_nope_head_dim, self.qk_rope_head_dim, self.v_head_dim,
                      self.rms_norm_eps, self.softmax_scale, self.rope_params(), self.dtype)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_weights(w: dict) -> Weights:
    ptrs = []
    for n in WEIGHT_NAMES:
        t = w.get(n) if n in OPTIONAL_WEIGHTS else w[n]
        if t is None:
            ptrs.append(None)
            continue
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"weight {n} must be a contiguous device tensor")
        ptrs.append(t.data_ptr())
    return Weights(*ptrs)


def mla_softmax_scale(cfg: MlaConfig) -> float:
    c = cfg.c()
    return float(load_library().mla_softmax_scale(ctypes.byref(c)))


def mla_version() -> str:
    return load_library().mla_version().decode()


PREFILL_STAGES = ("down_proj", "rmsnorm", "rope_k", "q_up_proj", "rope_q", "kv_up_proj",
                  "attention", "out_proj")
DECODE_STAGES = ("down_proj", "rmsnorm", "rope_k_append", "q_up_proj", "rope_q", "absorb",
                 "latent_attention", "split_merge", "unabsorb", "out_proj")


def mla_set_stage_events(events) -> None:
    """Record the given hipEvent_t handles (ints) at stage boundaries of the
    next prefill/decode calls on this thread; None switches it off."""
    lib = load_library()
    if not events:
        _check(lib.mla_set_stage_events(None, 0))
        mla_set_stage_events._keep = None
        return
    arr = (ctypes.c_void_p * len(events))(*events)
    mla_set_stage_events._keep = arr  # the library keeps the pointer
    _check(lib.mla_set_stage_events(arr, len(events)))


def mla_prefill_workspace_size(cfg: MlaConfig, batch: int, seq: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_prefill_workspace_size(ctypes.byref(c), batch, seq, ctypes.byref(n)))
    return n.value


def mla_prefill_layout_of(cfg: MlaConfig, batch: int, seq: int) -> PrefillLayout:
    lay = PrefillLayout()
    c = cfg.c()
    _check(load_library().mla_prefill_layout_of(ctypes.byref(c), batch, seq, ctypes.byref(lay)))
    return lay


def mla_decode_workspace_size(cfg: MlaConfig, batch: int, capacity: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_decode_workspace_size(ctypes.byref(c), batch, capacity,
                                                    ctypes.byref(n)))
    return n.value


def mla_decode_layout_of(cfg: MlaConfig, batch: int, capacity: int) -> DecodeLayout:
    lay = DecodeLayout()
    c = cfg.c()
    _check(load_library().mla_decode_layout_of(ctypes.byref(c), batch, capacity,
                                               ctypes.byref(lay)))
    return lay


def _device_check(*ts):
    for t in ts:
        if t is not None and not (t.is_cuda and t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def mla_prefill_forward(cfg: MlaConfig, weights: dict, x: torch.Tensor, y=None, latent_out=None,
                        workspace=None, stream=None, want_latent: bool = False):
    """y = MLA prefill of x [B, S, D].  Returns (y, latent_out, workspace)."""
    B, S, D = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((B, S, D), dtype=cfg.torch_dtype, device=dev)
    if latent_out is None and want_latent:
        latent_out = torch.empty((B, S, cfg.kv_lora_rank + cfg.qk_rope_head_dim),
                                 dtype=cfg.torch_dtype, device=dev)
    need = mla_prefill_workspace_size(cfg, B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _device_check(x, y, latent_out, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_prefill_forward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), B, S, _ptr(y), _ptr(latent_out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return y, latent_out, workspace


def mla_prefill_varlen_workspace_size(cfg: MlaConfig, n_seq: int, total_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_prefill_varlen_workspace_size(ctypes.byref(c), n_seq, total_tokens,
                                                            ctypes.byref(n)))
    return n.value


def mla_prefill_varlen_forward(cfg: MlaConfig, weights: dict, x: torch.Tensor,
                               cu_seqlens: torch.Tensor, y=None, latent_out=None, workspace=None,
                               stream=None, want_latent: bool = False):
    """Prefill of packed sequences: x [T, D], cu_seqlens int32 [n_seq + 1] on
    the device.  Returns (y [T, D], latent_out [T, r_kv + d_r], workspace)."""
    T, D = x.shape
    n_seq = cu_seqlens.numel() - 1
    dev = x.device
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if y is None:
        y = torch.empty((T, D), dtype=cfg.torch_dtype, device=dev)
    if latent_out is None and want_latent:
        latent_out = torch.empty((T, cfg.kv_lora_rank + cfg.qk_rope_head_dim),
                                 dtype=cfg.torch_dtype, device=dev)
    need = mla_prefill_varlen_workspace_size(cfg, n_seq, T)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _device_check(x, cu_seqlens, y, latent_out, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_prefill_varlen_forward(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), _ptr(cu_seqlens), n_seq, T, _ptr(y),
        _ptr(latent_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return y, latent_out, workspace


def mla_decode_absorbed(cfg: MlaConfig, weights: dict, x: torch.Tensor, latent_cache: torch.Tensor,
                        cache_lens: torch.Tensor, y=None, workspace=None, stream=None):
    """One absorbed decode step for x [B, D]; writes row lens[b] of the cache.
    Returns (y, workspace)."""
    B, D = x.shape
    cap = latent_cache.shape[1]
    dev = x.device
    if y is None:
        y = torch.empty((B, D), dtype=cfg.torch_dtype, device=dev)
    need = mla_decode_workspace_size(cfg, B, cap)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if cache_lens.dtype != torch.int32:
        raise ValueError("cache_lens must be int32")
    _device_check(x, y, latent_cache, cache_lens, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_decode_absorbed(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), B, _ptr(latent_cache), cap, _ptr(cache_lens),
        _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return y, workspace


def mla_decode_multi_workspace_size(cfg: MlaConfig, batch: int, q_len: int, capacity: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_decode_multi_workspace_size(ctypes.byref(c), batch, q_len, capacity,
                                                          ctypes.byref(n)))
    return n.value


def mla_decode_absorbed_multi(cfg: MlaConfig, weights: dict, x: torch.Tensor,
                              latent_cache: torch.Tensor, cache_lens: torch.Tensor, y=None,
                              workspace=None, stream=None):
    """Absorbed decode of q_len new tokens per sequence, x [B, q_len, D];
    writes cache rows lens[b] .. lens[b] + q_len - 1.  Returns (y, workspace)."""
    B, T, D = x.shape
    cap = latent_cache.shape[1]
    dev = x.device
    if y is None:
        y = torch.empty((B, T, D), dtype=cfg.torch_dtype, device=dev)
    need = mla_decode_multi_workspace_size(cfg, B, T, cap)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if cache_lens.dtype != torch.int32:
        raise ValueError("cache_lens must be int32")
    _device_check(x, y, latent_cache, cache_lens, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_decode_absorbed_multi(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), B, T, _ptr(latent_cache), cap,
        _ptr(cache_lens), _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return y, workspace


def mla_prefill_chunk_workspace_size(cfg: MlaConfig, batch: int, q_len: int, capacity: int,
                                     max_keys: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_prefill_chunk_workspace_size(ctypes.byref(c), batch, q_len, capacity,
                                                           max_keys, ctypes.byref(n)))
    return n.value


def mla_prefill_chunk(cfg: MlaConfig, weights: dict, x: torch.Tensor, latent_cache: torch.Tensor,
                      cache_lens: torch.Tensor, max_keys: int, y=None, workspace=None, stream=None):
    """Expanded-form prefill chunk, x [B, q_len, D] against the latent cache;
    writes cache rows lens[b] .. lens[b] + q_len - 1.  Returns (y, workspace)."""
    B, T, D = x.shape
    cap = latent_cache.shape[1]
    dev = x.device
    if y is None:
        y = torch.empty((B, T, D), dtype=cfg.torch_dtype, device=dev)
    need = mla_prefill_chunk_workspace_size(cfg, B, T, cap, max_keys)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if cache_lens.dtype != torch.int32:
        raise ValueError("cache_lens must be int32")
    _device_check(x, y, latent_cache, cache_lens, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_prefill_chunk(
        ctypes.byref(c), ctypes.byref(w), _ptr(x), B, T, _ptr(latent_cache), cap, _ptr(cache_lens),
        max_keys, _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return y, workspace


def mla_backward_workspace_size(cfg: MlaConfig, batch: int, seq: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_backward_workspace_size(ctypes.byref(c), batch, seq, ctypes.byref(n)))
    return n.value


def mla_backward(cfg: MlaConfig, weights: dict, x: torch.Tensor, dy: torch.Tensor, workspace=None,
                 stream=None):
    """Gradients of <dy, MLA(x)>: returns (dx, grads) with grads[name] shaped
    like weights[name] (cfg dtype; the RMSNorm gains' gradients fp32)."""
    B, S, D = x.shape
    if dy.shape != x.shape:
        raise ValueError(f"dy {tuple(dy.shape)} must have x's shape {tuple(x.shape)}")
    dev = x.device
    need = mla_backward_workspace_size(cfg, B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _device_check(x, dy, workspace)
    grads = {}
    for n in WEIGHT_NAMES:
        t = weights.get(n)
        if t is None:
            continue
        grads[n] = torch.empty(t.shape, dtype=torch.float32 if n in ("q_norm", "kv_norm") else cfg.torch_dtype,
                               device=dev)
    dx = torch.empty_like(x)
    g = WeightGrads(*[grads[n].data_ptr() if n in grads else None for n in WEIGHT_NAMES])
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_backward(ctypes.byref(c), ctypes.byref(w), _ptr(x), B, S, _ptr(dy), _ptr(dx),
                                       ctypes.byref(g), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))
    return dx, grads


def mla_attention_backward(q, k, v, o, dout, scale: float, workspace=None, stream=None):
    """(dq, dk, dv) of causal attention; q, k [..., S, d_qk], v, o, dout
    [..., S, d_v], contiguous, one dtype (fp32 or bf16)."""
    _check_attention_backward_shapes(q, k, v, o, dout)
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[q.dtype]
    S, dqk, dv_ = q.shape[-2], q.shape[-1], v.shape[-1]
    bh = q.numel() // max(S * dqk, 1)
    n = ctypes.c_size_t()
    _check(load_library().mla_attention_backward_workspace_size(bh, S, ctypes.byref(n)))
    if workspace is None:
        workspace = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dvt = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(load_library().mla_attention_backward(
        dt, bh, S, dqk, dv_, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dvt), _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dvt


def _check_attention_backward_shapes(q, k, v, o, dout):
    ts = (q, k, v, o, dout)
    # only q's S and d_qk and v's d_v reach the library: every other shape
    # must follow from them, or the kernels would read past the buffers
    if q.dim() < 2 or k.shape != q.shape:
        raise ValueError(f"k {tuple(k.shape)} must have q's shape {tuple(q.shape)}")
    if v.shape[:-1] != q.shape[:-1]:
        raise ValueError(f"v {tuple(v.shape)} must match q {tuple(q.shape)} but for the last axis")
    if o.shape != v.shape or dout.shape != v.shape:
        raise ValueError(f"o {tuple(o.shape)} and dout {tuple(dout.shape)} must have v's shape "
                         f"{tuple(v.shape)}")
    if any(not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype for t in ts):
        raise ValueError("q, k, v, o and dout must be contiguous device tensors of one dtype")


def mla_attention_backward_noalloc_max_rows() -> int:
    """Rows (batch_heads x seq) the allocation-free backward's built-in
    scratch holds."""
    return int(load_library().mla_attention_backward_noalloc_max_rows())


def mla_attention_backward_noalloc(q, k, v, o, dout, scale: float, dq=None, dk=None, dv=None,
                                   stream=None):
    """mla_attention_backward without a workspace (the library's built-in
    scratch); the outputs may be passed in, so the call need not allocate."""
    _check_attention_backward_shapes(q, k, v, o, dout)
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[q.dtype]
    S, dqk, dv_ = q.shape[-2], q.shape[-1], v.shape[-1]
    bh = q.numel() // max(S * dqk, 1)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous device tensors shaped like q, k, v")
    _check(load_library().mla_attention_backward_noalloc(
        dt, bh, S, dqk, dv_, scale, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), _stream(stream)))
    return dq, dk, dv


def mla_rmsnorm_backward(x, dy, g, eps: float, stream=None):
    """(dx, dg) of the RMSNorm y = x r g over the last axis; x, dy [rows, n]
    and g [n] contiguous device tensors of one dtype; dg is fp32."""
    if x.dim() < 1 or dy.shape != x.shape:
        raise ValueError(f"dy {tuple(dy.shape)} must have x's shape {tuple(x.shape)}")
    if g.shape != (x.shape[-1],):
        raise ValueError(f"g {tuple(g.shape)} must be ({x.shape[-1]},)")
    if any(not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype for t in (x, dy, g)):
        raise ValueError("x, dy and g must be contiguous device tensors of one dtype")
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[x.dtype]
    n = x.shape[-1]
    rows = x.numel() // n
    dx = torch.empty_like(x)
    dg = torch.empty(n, dtype=torch.float32, device=x.device)
    need = ctypes.c_size_t(0)
    _check(load_library().mla_rmsnorm_backward_workspace_size(rows, n, ctypes.byref(need)))
    ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=x.device)
    _check(load_library().mla_rmsnorm_backward(dt, _ptr(x), _ptr(dy), _ptr(g), rows, n, eps, _ptr(dx), _ptr(dg),
                                               _ptr(ws), ws.numel(), _stream(stream)))
    return dx, dg


def mla_fp8_prepare_weights(cfg: MlaConfig, weights: dict, stream=None):
    """Block-quantise the bf16 projection weights for mla_prefill_forward_fp8.
    Returns (buffer, Fp8Weights): the device buffer owns the codes and scale
    bytes; keep it alive while the struct is used."""
    lib = load_library()
    c = cfg.c()
    n = ctypes.c_size_t(0)
    _check(lib.mla_fp8_weights_size(ctypes.byref(c), ctypes.byref(n)))
    dev = next(iter(weights.values())).device
    buf = torch.empty(n.value, dtype=torch.uint8, device=dev)
    w = make_weights(weights)
    w8 = Fp8Weights()
    _check(lib.mla_fp8_prepare_weights(ctypes.byref(c), ctypes.byref(w), _ptr(buf), n.value, ctypes.byref(w8),
                                       _stream(stream)))
    return buf, w8


def mla_prefill_fp8_workspace_size(cfg: MlaConfig, batch: int, seq: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(load_library().mla_prefill_fp8_workspace_size(ctypes.byref(c), batch, seq, ctypes.byref(n)))
    return n.value


def mla_prefill_forward_fp8(cfg: MlaConfig, weights: dict, w8: Fp8Weights, x: torch.Tensor, y=None,
                            latent_out=None, workspace=None, stream=None, want_latent: bool = False):
    """The prefill with FP8 projections (w8 from mla_fp8_prepare_weights; from
    `weights` only q_norm and the optional kv_norm are read).  Returns
    (y, latent_out, workspace)."""
    B, S, D = x.shape
    dev = x.device
    if y is None:
        y = torch.empty((B, S, D), dtype=cfg.torch_dtype, device=dev)
    if latent_out is None and want_latent:
        latent_out = torch.empty((B, S, cfg.kv_lora_rank + cfg.qk_rope_head_dim), dtype=cfg.torch_dtype,
                                 device=dev)
    need = mla_prefill_fp8_workspace_size(cfg, B, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _device_check(x, y, latent_out, workspace)
    w = make_weights(weights)
    c = cfg.c()
    _check(load_library().mla_prefill_forward_fp8(
        ctypes.byref(c), ctypes.byref(w), ctypes.byref(w8), _ptr(x), B, S, _ptr(y), _ptr(latent_out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return y, latent_out, workspace


def mla_fp8_scale_pitch(rows: int) -> int:
    """Row pitch of the scale bytes that mla_fp8_gemm takes for `rows` rows."""
    return int(load_library().mla_fp8_scale_pitch(rows))


def _fp8_quantize(fn, x: torch.Tensor, q_align: int, stream):
    if x.dim() != 2 or x.stride(-1) != 1 or not x.is_cuda:
        raise ValueError("x must be a device [rows, cols] tensor with unit last stride")
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[x.dtype]
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    pitch = mla_fp8_scale_pitch(rows)
    sexp = torch.empty((max(cols // 128, 1), pitch), dtype=torch.uint8, device=x.device)
    _check(fn(_ptr(x), dt, rows, cols, x.stride(0), _ptr(q), q.stride(0), _ptr(sexp), pitch, _stream(stream)))
    return q, sexp


def mla_fp8_quantize_rows(x: torch.Tensor, stream=None):
    """1 x 128 activation tiles of x [rows, cols] (fp32/bf16) -> (codes uint8
    [rows, cols], scale bytes uint8 [cols / 128, mla_fp8_scale_pitch(rows)])."""
    return _fp8_quantize(load_library().mla_fp8_quantize_rows, x, 2, stream)


def mla_fp8_quantize_blocks(w: torch.Tensor, stream=None):
    """128 x 128 weight blocks of w [rows, cols] -> (codes, scale bytes), the
    block's byte repeated on each of its rows."""
    return _fp8_quantize(load_library().mla_fp8_quantize_blocks, w, 16, stream)


def mla_fp8_gemm(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                 out_dtype=torch.bfloat16, c: Optional[torch.Tensor] = None, stream=None):
    """C [M, N] = block-scaled a [M, K] times block-scaled b [N, K] transposed."""
    for t in (a, sa, b, sb):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.stride(-1) != 1 or not t.is_cuda:
            raise ValueError("a, sa, b and sb must be device uint8 matrices with unit last stride")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or sa.shape[0] * 128 < K or sb.shape[0] * 128 < K:
        raise ValueError("inner dimensions do not match")
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=a.device)
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[c.dtype]
    _check(load_library().mla_fp8_gemm(_ptr(a), a.stride(0), _ptr(sa), sa.stride(0), _ptr(b), b.stride(0),
                                       _ptr(sb), sb.stride(0), _ptr(c), dt, c.stride(0), M, N, K,
                                       _stream(stream)))
    return c


def mla_rope_apply(x: torch.Tensor, positions: torch.Tensor, params: RopeParams, stream=None):
    """In-place RoPE of x [n_tokens, n_heads, rope_dim] (any strides, unit
    stride on the last axis) at positions [n_tokens] int32."""
    if x.dim() != 3 or x.stride(-1) != 1:
        raise ValueError("x must be [n_tokens, n_heads, rope_dim] with unit last stride")
    if positions.dtype != torch.int32 or not positions.is_cuda:
        raise ValueError("positions must be a device int32 tensor")
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[x.dtype]
    n, h, d = x.shape
    _check(load_library().mla_rope_apply(
        _ptr(x), dt, n, h, d, x.stride(0), x.stride(1), _ptr(positions), ctypes.byref(params),
        _stream(stream)))
    return x
