// Layout and reduction helpers of the MLA backward (gfx950): moves between
// the head-major per-head tensors the attention kernels use and the
// token-major rows the projection products use, the keys' assembly, the sum
// of the shared RoPE key's gradient over heads, and the negated positions of
// the RoPE backward.  All bandwidth-bound: one 16-byte chunk per thread
// (every width and column offset here is a multiple of 8 elements, checked
// by the caller's config rules).

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

template <typename T> constexpr int vec_of() { return 16 / (int)sizeof(T); }

// dst[(b S + s) ldd + dcol + h w + c] = src[((b H + h) S + s) sp + scol + c],
// c < w; to_heads swaps the roles (src token-major, dst head-major).
template <typename T, bool TO_HEADS>
__global__ __launch_bounds__(256) void permute_heads_kernel(const T *src, int64_t sp, int scol, T *dst,
                                                            int64_t dp, int dcol, int w, int B, int S,
                                                            int H) {
  constexpr int V = vec_of<T>();
  const int cpw = w / V;
  const int64_t n = (int64_t)B * S * H * cpw;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i % cpw) * V;
    const int64_t r = i / cpw;           // (b, s, h) with h fastest
    const int h = (int)(r % H);
    const int64_t t = r / H;             // token b S + s
    const int b = (int)(t / S), s = (int)(t % S);
    const int64_t hrow = ((int64_t)b * H + h) * S + s;
    const T *from;
    T *to;
    if constexpr (TO_HEADS) {
      from = src + t * sp + scol + (int64_t)h * w + c;
      to = dst + hrow * dp + dcol + c;
    } else {
      from = src + hrow * sp + scol + c;
      to = dst + t * dp + dcol + (int64_t)h * w + c;
    }
    *reinterpret_cast<uint4 *>(to) = *reinterpret_cast<const uint4 *>(from);
  }
}

// K_h = [k_nope_h ‖ k_pe]: kh [B, H, S, dn + dr] from k_nope [B, H, S, dn]
// and the shared k_pe rows (pitch ld_kpe, token b S + s).
template <typename T>
__global__ __launch_bounds__(256) void build_keys_kernel(const T *kn, const T *kpe, int64_t ld_kpe, T *kh,
                                                         int dn, int dr, int B, int S, int H) {
  constexpr int V = vec_of<T>();
  const int cpr = (dn + dr) / V;
  const int64_t n = (int64_t)B * H * S * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i % cpr) * V;
    const int64_t hrow = i / cpr;  // (b H + h) S + s
    const int s = (int)(hrow % S);
    const int b = (int)(hrow / S / H);
    const T *from = c < dn ? kn + hrow * dn + c : kpe + ((int64_t)b * S + s) * ld_kpe + (c - dn);
    *reinterpret_cast<uint4 *>(kh + hrow * (dn + dr) + c) = *reinterpret_cast<const uint4 *>(from);
  }
}

// dst[(b S + s) ldd + c] = sum over h = 0..H-1 (in order) of
// src[((b H + h) S + s) sp + scol + c], fp32 sums; one element per thread.
template <typename T>
__global__ __launch_bounds__(256) void head_sum_kernel(const T *src, int64_t sp, int scol, T *dst, int64_t ldd,
                                                       int w, int B, int S, int H) {
  const int64_t n = (int64_t)B * S * w;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i % w);
    const int64_t t = i / w;
    const int b = (int)(t / S), s = (int)(t % S);
    float acc = 0.f;
    for (int h = 0; h < H; ++h) acc += to_f32(src[(((int64_t)b * H + h) * S + s) * sp + scol + c]);
    dst[t * ldd + c] = from_f32<T>(acc);
  }
}

// 64 x 64 tiles through LDS: 16-byte loads of source rows, 16-byte stores of
// destination rows (each gathered from eight LDS rows; the 144-byte pitch
// puts those eight 2-byte reads in distinct banks).
__global__ __launch_bounds__(256) void transpose_kernel(const bf16 *src, int64_t lds, int R, int C, bf16 *dst,
                                                        int64_t ldd) {
  __shared__ __attribute__((aligned(16))) bf16 t[64][72];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = tid + 256 * i;  // source row ch / 8, columns 8 (ch % 8) ..
    const int r = ch >> 3, c = (ch & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < R && c0 + c < C) v = *reinterpret_cast<const uint4 *>(src + (int64_t)(r0 + r) * lds + c0 + c);
    *reinterpret_cast<uint4 *>(&t[r][c]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = tid + 256 * i;  // destination row (source column) ch / 8, its columns 8 (ch % 8) ..
    const int c = ch >> 3, r = (ch & 7) * 8;
    if (c0 + c < C && r0 + r < R) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = t[r + e][c];
      *reinterpret_cast<bf16x8 *>(dst + (int64_t)(c0 + c) * ldd + r0 + r) = v;
    }
  }
}

__global__ __launch_bounds__(256) void neg_positions_kernel(int32_t *pos, int64_t n, int S) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) pos[t] = -(int32_t)(t % S);
}

unsigned grid_for(int64_t items) {
  const int64_t g = (items + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_permute_heads(int dtype, bool to_heads, const void *src, int64_t sp, int scol, void *dst,
                                int64_t dp, int dcol, int w, int B, int S, int H, hipStream_t st) {
  const int64_t items = (int64_t)B * S * H * (w / (dtype == BF16 ? 8 : 4));
  if (items == 0) return hipSuccess;
  const unsigned g = grid_for(items);
#define MLA_PERM(T_, TO_)                                                                                \
  hipLaunchKernelGGL((permute_heads_kernel<T_, TO_>), dim3(g), dim3(256), 0, st,                         \
                     reinterpret_cast<const T_ *>(src), sp, scol, reinterpret_cast<T_ *>(dst), dp, dcol, w, B, \
                     S, H)
  if (dtype == BF16) {
    if (to_heads) MLA_PERM(bf16, true); else MLA_PERM(bf16, false);
  } else {
    if (to_heads) MLA_PERM(float, true); else MLA_PERM(float, false);
  }
#undef MLA_PERM
  return hipGetLastError();
}

hipError_t launch_build_keys(int dtype, const void *kn, const void *kpe, int64_t ld_kpe, void *kh, int dn, int dr,
                             int B, int S, int H, hipStream_t st) {
  const int64_t items = (int64_t)B * H * S * ((dn + dr) / (dtype == BF16 ? 8 : 4));
  if (items == 0) return hipSuccess;
  if (dtype == BF16)
    hipLaunchKernelGGL(build_keys_kernel<bf16>, dim3(grid_for(items)), dim3(256), 0, st,
                       reinterpret_cast<const bf16 *>(kn), reinterpret_cast<const bf16 *>(kpe), ld_kpe,
                       reinterpret_cast<bf16 *>(kh), dn, dr, B, S, H);
  else
    hipLaunchKernelGGL(build_keys_kernel<float>, dim3(grid_for(items)), dim3(256), 0, st,
                       reinterpret_cast<const float *>(kn), reinterpret_cast<const float *>(kpe), ld_kpe,
                       reinterpret_cast<float *>(kh), dn, dr, B, S, H);
  return hipGetLastError();
}

hipError_t launch_head_sum(int dtype, const void *src, int64_t sp, int scol, void *dst, int64_t ldd, int w, int B,
                           int S, int H, hipStream_t st) {
  const int64_t items = (int64_t)B * S * w;
  if (items == 0) return hipSuccess;
  if (dtype == BF16)
    hipLaunchKernelGGL(head_sum_kernel<bf16>, dim3(grid_for(items)), dim3(256), 0, st,
                       reinterpret_cast<const bf16 *>(src), sp, scol, reinterpret_cast<bf16 *>(dst), ldd, w, B, S,
                       H);
  else
    hipLaunchKernelGGL(head_sum_kernel<float>, dim3(grid_for(items)), dim3(256), 0, st,
                       reinterpret_cast<const float *>(src), sp, scol, reinterpret_cast<float *>(dst), ldd, w, B,
                       S, H);
  return hipGetLastError();
}

hipError_t launch_transpose(const void *src, int64_t lds, int R, int C, void *dst, int64_t ldd, hipStream_t st) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (R % 8 || C % 8 || lds % 8 || ldd % 8 || ((uintptr_t)src | (uintptr_t)dst) % 16 || (R + 63) / 64 > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)), dim3(256), 0, st,
                     reinterpret_cast<const bf16 *>(src), lds, R, C, reinterpret_cast<bf16 *>(dst), ldd);
  return hipGetLastError();
}

hipError_t launch_neg_positions(int32_t *pos, int64_t n, int S, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(neg_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pos, n, S);
  return hipGetLastError();
}

}  // namespace mla
