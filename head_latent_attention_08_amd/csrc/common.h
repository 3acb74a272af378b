// Device-side building blocks shared by the MLA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// 32x32 MFMA tile traits.  A lane l holds, for the A operand, row l%32 and
// KPL consecutive k values starting at (l/32)*KPL; for B, column l%32 and
// the same k values; the accumulator element r of lane l is row
// (r/4)*8 + (l/32)*4 + r%4, column l%32.  A dot product over k is the same
// for any k order shared by A and B, which the attention kernels use to
// feed accumulator values straight back as an operand.
template <typename T> struct Mfma32;

template <> struct Mfma32<bf16> {
  static constexpr int KPL = 8;   // k values per lane
  static constexpr int KSTEP = 16;
  using frag = bf16x8;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma32<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  using frag = float;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// 16x16 MFMA tile traits (same conventions): A lane l holds row l%16 and
// KPL k values from (l/16)*KPL; B lane l holds column l%16 and the same k
// values; accumulator element r of lane l is row (l/16)*4 + r, column l%16.
template <typename T> struct Mfma16;

template <> struct Mfma16<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 32;
  using frag = bf16x8;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma16<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 4;
  using frag = float;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline int acc_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

template <typename T> __device__ inline float to_f32(T v) { return (float)v; }

// One RoPE rotation (a, b) -> (a cos - b sin, b cos + a sin) with a fixed
// rounding (each product with sin rounded, then one fused multiply-add), so
// that the rotation kernels and a GEMM epilogue that rotates its output
// give the same bits.
__device__ inline void rope_rot(float a, float b, float c, float s, float &ra, float &rb) {
  ra = fmaf(a, c, -(b * s));
  rb = fmaf(b, c, a * s);
}
template <typename T> __device__ inline T from_f32(float v) { return (T)v; }

// 16-byte vector of T.
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
};

// max / sum of v over lanes l and l ^ 32, in every lane: one VALU lane swap
// between the wave's halves (v_permlane32_swap) instead of an LDS permute.
__device__ inline float half_swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace mla
