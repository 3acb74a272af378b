// Bandwidth-bound helpers of the MLA forward: RMSNorm of c_q, RoPE in both
// conventions, latent-row copies and the decode cache append.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

// RMSNorm: one wave per row, fp32 sum of squares, x * rsqrt(mean + eps) * g.
// Rows are read in 16-byte chunks (n and the row stride are multiples of 8
// elements and rows 16-byte aligned, checked on the host); the chunks a lane
// owns are loaded together so their latencies overlap.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(T *x, int64_t rows, int64_t ld, int n,
                                                      const T *g, float eps) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int UNR = 4;  // chunks in flight per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  T *xr = x + row * ld;
  const int nch = n / VEC;
  float ss = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64 * UNR) {
    uint4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = c0 + u * 64 + lane;
      v[u] = c < nch ? *reinterpret_cast<const uint4 *>(xr + c * VEC) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const T *e = reinterpret_cast<const T *>(&v[u]);
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float f = to_f32(e[k]);
        ss += f * f;
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)n + eps);
  for (int c0 = 0; c0 < nch; c0 += 64 * UNR) {
    uint4 v[UNR], w[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
        v[u] = *reinterpret_cast<const uint4 *>(xr + c * VEC);
        w[u] = *reinterpret_cast<const uint4 *>(g + c * VEC);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < nch) {
        T o[VEC];
        const T *e = reinterpret_cast<const T *>(&v[u]), *ge = reinterpret_cast<const T *>(&w[u]);
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = from_f32<T>(to_f32(e[k]) * inv * to_f32(ge[k]));
        *reinterpret_cast<uint4 *>(xr + c * VEC) = *reinterpret_cast<const uint4 *>(o);
      }
    }
  }
}

// RoPE.  A workgroup takes `tpb` consecutive tokens: it first forms
// cos/sin of every (token, pair) in float64 (the angle pos * inv_freq is
// reduced in double precision, so large positions keep full accuracy), then
// rotates all heads of those tokens.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T *x, int64_t n_tok, int64_t S, int64_t sb,
                                                   int64_t ss, int n_heads, int64_t sh,
                                                   const int32_t *positions, RopeTab tab,
                                                   int tpb, float *tab_out) {
  __shared__ float cs[256], sn[256];
  const int P = tab.pairs;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int i = threadIdx.x; i < tpb * P; i += blockDim.x) {
    const int64_t t = t0 + i / P;
    if (t < n_tok) {
      const int pr = i % P;
      const double pos = positions ? (double)positions[t] : (double)(t % S);
      double s, c;
      sincos(pos * tab.inv_freq[pr], &s, &c);
      cs[i] = (float)c * tab.amp;
      sn[i] = (float)s * tab.amp;
      if (tab_out && blockIdx.y == 0) {
        tab_out[t * 2 * P + pr] = cs[i];
        tab_out[t * 2 * P + P + pr] = sn[i];
      }
    }
  }
  __syncthreads();
  const int per_tok = n_heads * P;
  for (int i = threadIdx.x; i < tpb * per_tok; i += blockDim.x) {
    const int tl = i / per_tok;
    const int64_t t = t0 + tl;
    if (t >= n_tok) break;
    const int rem = i - tl * per_tok;
    const int h = rem / P, pr = rem - h * P;
    T *base = x + (t / S) * sb + (t % S) * ss + (int64_t)h * sh;
    const int i0 = tab.convention == 0 ? pr : 2 * pr;
    const int i1 = tab.convention == 0 ? pr + P : 2 * pr + 1;
    const float a = to_f32(base[i0]), b = to_f32(base[i1]);
    float ra, rb;
    rope_rot(a, b, cs[tl * P + pr], sn[tl * P + pr], ra, rb);
    base[i0] = from_f32<T>(ra);
    base[i1] = from_f32<T>(rb);
  }
}

// RoPE with 16-byte accesses: a thread rotates 8 pairs of one (token, head),
// held in two 16-byte chunks -- elements 16c..16c+15 (interleaved pairs) or
// 8c..8c+7 with their partners 8c+P..8c+P+7 (half-split).  Needs rope_dim a
// multiple of 16 and 16-byte aligned rows (checked on the host).  Blocks take
// tpb tokens (all heads) or, for many heads, one token and a range of heads
// (grid y); the cos/sin of the block's tokens are formed in float64 first.
template <typename T>
__global__ __launch_bounds__(256) void rope_vec_kernel(T *x, int64_t n_tok, int64_t S, int64_t sb,
                                                       int64_t ss, int n_heads, int64_t sh,
                                                       const int32_t *positions, RopeTab tab,
                                                       int tpb, float *tab_out) {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "16-byte chunks of bf16 or fp32");
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float cs[256], sn[256];
  const int P = tab.pairs, CH = P / 8;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int i = threadIdx.x; i < tpb * P; i += blockDim.x) {
    const int64_t t = t0 + i / P;
    if (t < n_tok) {
      const int pr = i % P;
      const double pos = positions ? (double)positions[t] : (double)(t % S);
      double s, c;
      sincos(pos * tab.inv_freq[pr], &s, &c);
      cs[i] = (float)c * tab.amp;
      sn[i] = (float)s * tab.amp;
      if (tab_out && blockIdx.y == 0) {
        tab_out[t * 2 * P + pr] = cs[i];
        tab_out[t * 2 * P + P + pr] = sn[i];
      }
    }
  }
  __syncthreads();
  const int per_tok = n_heads * CH;
  const int i = blockIdx.y * blockDim.x + threadIdx.x;
  const int tl = i / per_tok;
  const int64_t t = t0 + tl;
  if (tl >= tpb || t >= n_tok) return;
  const int rem = i - tl * per_tok;
  const int h = rem / CH, c = rem - h * CH;
  T *base = x + (t / S) * sb + (t % S) * ss + (int64_t)h * sh;
  const float *ct = cs + tl * P, *st = sn + tl * P;
  if (tab.convention == 0) {
    // pairs (8c + k, 8c + k + P), k < 8
    T a[8], b[8];
#pragma unroll
    for (int q = 0; q < 8 / VEC; ++q) {
      *reinterpret_cast<uint4 *>(a + q * VEC) = *reinterpret_cast<const uint4 *>(base + 8 * c + q * VEC);
      *reinterpret_cast<uint4 *>(b + q * VEC) = *reinterpret_cast<const uint4 *>(base + 8 * c + P + q * VEC);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float ra, rb;
      rope_rot(to_f32(a[k]), to_f32(b[k]), ct[8 * c + k], st[8 * c + k], ra, rb);
      a[k] = from_f32<T>(ra);
      b[k] = from_f32<T>(rb);
    }
#pragma unroll
    for (int q = 0; q < 8 / VEC; ++q) {
      *reinterpret_cast<uint4 *>(base + 8 * c + q * VEC) = *reinterpret_cast<const uint4 *>(a + q * VEC);
      *reinterpret_cast<uint4 *>(base + 8 * c + P + q * VEC) = *reinterpret_cast<const uint4 *>(b + q * VEC);
    }
  } else {
    // pairs (16c + 2k, 16c + 2k + 1), k < 8
    T v[16];
#pragma unroll
    for (int q = 0; q < 16 / VEC; ++q)
      *reinterpret_cast<uint4 *>(v + q * VEC) = *reinterpret_cast<const uint4 *>(base + 16 * c + q * VEC);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float ra, rb;
      rope_rot(to_f32(v[2 * k]), to_f32(v[2 * k + 1]), ct[8 * c + k], st[8 * c + k], ra, rb);
      v[2 * k] = from_f32<T>(ra);
      v[2 * k + 1] = from_f32<T>(rb);
    }
#pragma unroll
    for (int q = 0; q < 16 / VEC; ++q)
      *reinterpret_cast<uint4 *>(base + 16 * c + q * VEC) = *reinterpret_cast<const uint4 *>(v + q * VEC);
  }
}

template <typename T>
__global__ void copy_rows_kernel(T *dst, int64_t ldd, const T *src, int64_t lds, int64_t rows,
                                 int width) {
  const int64_t total = rows * width;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / width;
    const int c = (int)(i - r * width);
    dst[r * ldd + c] = src[r * lds + c];
  }
}

// The same copy in 16-byte chunks (widths, pitches and both bases a whole
// number of chunks): a workgroup takes one row block of 256 / nch rows.
__global__ __launch_bounds__(256) void copy_rows16_kernel(uint4 *dst, int64_t ldd, const uint4 *src,
                                                          int64_t lds, int64_t rows, int nch) {
  const int64_t total = rows * nch;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nch;
    const int c = (int)(i - r * nch);
    dst[r * ldd + c] = src[r * lds + c];
  }
}

template <typename T>
__global__ void cache_append_kernel(T *cache, int64_t cap, const int32_t *lens, int q_len,
                                    const T *src, int64_t lds, int width) {
  const int row = blockIdx.x, b = row / q_len, t = row - b * q_len;
  const int32_t L = lens[b];
  if (L < 0 || (int64_t)L + q_len > cap) return;
  T *dst = cache + ((int64_t)b * cap + L + t) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) dst[c] = src[(int64_t)row * lds + c];
}

__global__ void decode_positions_kernel(const int32_t *lens, int n, int q_len, int32_t *pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) pos[i] = lens[i / q_len] + i % q_len;
}

}  // namespace

hipError_t launch_rmsnorm(int dtype, void *x, int64_t rows, int64_t ld, int n, const void *g,
                          float eps, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (dtype == BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16>, grid, dim3(256), 0, st, (bf16 *)x, rows, ld, n,
                       (const bf16 *)g, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, grid, dim3(256), 0, st, (float *)x, rows, ld, n,
                       (const float *)g, eps);
  return hipGetLastError();
}

hipError_t launch_rope(int dtype, void *x, int64_t n_tok, int64_t S, int64_t sb, int64_t ss,
                       int n_heads, int64_t sh, const int32_t *positions, const RopeTab &tab,
                       hipStream_t st, float *tab_out) {
  if (n_tok <= 0) return hipSuccess;
  const int64_t vec = dtype == BF16 ? 8 : 4;
  const bool vector = tab.pairs % 8 == 0 && ((uintptr_t)x & 15) == 0 && sb % vec == 0 &&
                      ss % vec == 0 && sh % vec == 0 && tab.pairs <= 256;
  if (vector) {
    const int per_tok = n_heads * (tab.pairs / 8);
    int tpb = per_tok >= 256 ? 1 : 256 / per_tok;
    if (tpb * tab.pairs > 256) tpb = 256 / tab.pairs;
    if (tpb < 1) tpb = 1;
    dim3 grid((unsigned)((n_tok + tpb - 1) / tpb), (unsigned)((tpb * per_tok + 255) / 256));
    if (dtype == BF16)
      hipLaunchKernelGGL(rope_vec_kernel<bf16>, grid, dim3(256), 0, st, (bf16 *)x, n_tok, S, sb,
                         ss, n_heads, sh, positions, tab, tpb, tab_out);
    else
      hipLaunchKernelGGL(rope_vec_kernel<float>, grid, dim3(256), 0, st, (float *)x, n_tok, S,
                         sb, ss, n_heads, sh, positions, tab, tpb, tab_out);
    return hipGetLastError();
  }
  int per_tok = n_heads * tab.pairs;
  int tpb = per_tok >= 256 ? 1 : 256 / per_tok;
  if (tpb * tab.pairs > 256) tpb = 256 / tab.pairs;
  if (tpb < 1) tpb = 1;
  dim3 grid((unsigned)((n_tok + tpb - 1) / tpb));
  if (dtype == BF16)
    hipLaunchKernelGGL(rope_kernel<bf16>, grid, dim3(256), 0, st, (bf16 *)x, n_tok, S, sb, ss,
                       n_heads, sh, positions, tab, tpb, tab_out);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(256), 0, st, (float *)x, n_tok, S, sb, ss,
                       n_heads, sh, positions, tab, tpb, tab_out);
  return hipGetLastError();
}

namespace {
// Token t of a packed stream: the first token of its sequence (the largest b
// with cu[b] <= t; cu is non-decreasing when valid), which is the first key
// t attends (the last is t itself), and its position in the sequence.  The
// start is clamped into [0, t] so that every later access stays in range
// even for invalid offsets; valid[t] copies the check's verdict.
__global__ __launch_bounds__(256) void varlen_index_kernel(const int32_t *cu, int n_seq, int64_t T,
                                                           int32_t *start, int32_t *last,
                                                           int32_t *pos, int32_t *valid,
                                                           const int32_t *ok) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  int64_t s0 = cu[lo];
  s0 = s0 < 0 ? 0 : (s0 > t ? t : s0);
  start[t] = (int32_t)s0;
  last[t] = (int32_t)t;
  pos[t] = (int32_t)(t - s0);
  valid[t] = ok[0];
}

// valid[0] = 1 when cu[0] = 0, cu is non-decreasing and cu[n_seq] = T, else 0
// (one workgroup).
__global__ __launch_bounds__(256) void varlen_check_kernel(const int32_t *cu, int n_seq, int64_t T,
                                                           int32_t *valid) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (cu[0] != 0 || (int64_t)cu[n_seq] != T) ? 1 : 0;
  __syncthreads();
  int mine = 0;
  for (int b = threadIdx.x; b < n_seq; b += 256) mine |= cu[b] > cu[b + 1] ? 1 : 0;
  if (mine) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) valid[0] = bad ? 0 : 1;
}
}  // namespace

hipError_t launch_varlen_index(const int32_t *cu_seqlens, int n_seq, int64_t total, int32_t *start,
                               int32_t *last, int32_t *pos, int32_t *valid, int32_t *ok,
                               hipStream_t st) {
  if (n_seq <= 0 || total <= 0) return hipSuccess;
  hipLaunchKernelGGL(varlen_check_kernel, dim3(1), dim3(256), 0, st, cu_seqlens, n_seq, total, ok);
  hipLaunchKernelGGL(varlen_index_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     cu_seqlens, n_seq, total, start, last, pos, valid, ok);
  return hipGetLastError();
}

namespace {
// Chunk of q_len tokens per sequence against a latent cache, key stream side
// (one workgroup): sequence b is usable when 0 <= L_b and L_b + q_len <= cap;
// its keys are its L_b + q_len cache rows, packed at kofs[b] (kofs[B] = all
// keys).  When the keys do not fit max_keys no sequence is usable.
// lens_eff[b] = L_b for a usable sequence, else -1 (no keys, no cache write).
__global__ __launch_bounds__(256) void chunk_scan_kernel(const int32_t *lens, int B, int q_len,
                                                         int64_t cap, int64_t max_keys,
                                                         int32_t *lens_eff, int32_t *kofs) {
  __shared__ int64_t part[256];
  const int per = (B + 255) / 256, b0 = threadIdx.x * per;
  int64_t sum = 0;
  for (int b = b0; b < min(B, b0 + per); ++b) {
    const int64_t L = lens[b];
    if (L >= 0 && L + q_len <= cap) sum += L + q_len;
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  // inclusive scan of the 256 partial sums (Hillis-Steele)
  for (int d = 1; d < 256; d *= 2) {
    const int64_t v = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  const bool fits = part[255] <= max_keys;
  int64_t run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
  for (int b = b0; b < min(B, b0 + per); ++b) {
    const int64_t L = lens[b];
    const bool ok = fits && L >= 0 && L + q_len <= cap;
    kofs[b] = (int32_t)(fits ? run : 0);
    lens_eff[b] = ok ? (int32_t)L : -1;
    if (ok) run += L + q_len;
  }
  if (threadIdx.x == 255) kofs[B] = (int32_t)(fits ? part[255] : 0);
}

// Query b * q_len + t: keys kofs[b] .. kofs[b] + L_b + t of the stream (an
// empty range for an unusable sequence), position L_b + t, validity.
__global__ __launch_bounds__(256) void chunk_ranges_kernel(const int32_t *lens_eff, const int32_t *kofs,
                                                           int n, int q_len, int32_t *lo, int32_t *hi,
                                                           int32_t *pos, int32_t *valid) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int b = i / q_len, t = i - b * q_len;
  const int L = lens_eff[b];
  lo[i] = kofs[b];
  hi[i] = L >= 0 ? kofs[b] + L + t : kofs[b] - 1;
  pos[i] = L >= 0 ? L + t : t;
  valid[i] = L >= 0 ? 1 : 0;
}

// Key stream row k: row k - kofs[b] of sequence b's cache (the sequence
// whose packed range holds k), or zeros past the last key.
template <typename T>
__global__ __launch_bounds__(256) void gather_keys_kernel(T *dst, int64_t n_rows, const T *cache,
                                                          int64_t cap, int width, const int32_t *kofs,
                                                          int B) {
  const int64_t k = blockIdx.x;
  if (k >= n_rows) return;
  T *out = dst + k * width;
  if (k >= kofs[B]) {
    for (int c = threadIdx.x; c < width; c += blockDim.x) out[c] = from_f32<T>(0.f);
    return;
  }
  int lo = 0, hi = B - 1;  // the last b with kofs[b] <= k
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (kofs[mid] <= k) lo = mid;
    else hi = mid - 1;
  }
  const T *src = cache + ((int64_t)lo * cap + (k - kofs[lo])) * width;
  for (int c = threadIdx.x; c < width; c += blockDim.x) out[c] = src[c];
}
}  // namespace

hipError_t launch_chunk_index(const int32_t *lens, int B, int q_len, int64_t cap, int64_t max_keys,
                              int32_t *lens_eff, int32_t *kofs, int32_t *lo, int32_t *hi, int32_t *pos,
                              int32_t *valid, hipStream_t st) {
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(256), 0, st, lens, B, q_len, cap, max_keys, lens_eff,
                     kofs);
  const int n = B * q_len;
  hipLaunchKernelGGL(chunk_ranges_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, lens_eff, kofs,
                     n, q_len, lo, hi, pos, valid);
  return hipGetLastError();
}

hipError_t launch_gather_keys(int dtype, void *dst, int64_t n_rows, const void *cache, int64_t cap,
                              int width, const int32_t *kofs, int B, hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  if (dtype == BF16)
    hipLaunchKernelGGL(gather_keys_kernel<bf16>, dim3((unsigned)n_rows), dim3(256), 0, st, (bf16 *)dst, n_rows,
                       (const bf16 *)cache, cap, width, kofs, B);
  else
    hipLaunchKernelGGL(gather_keys_kernel<float>, dim3((unsigned)n_rows), dim3(256), 0, st, (float *)dst,
                       n_rows, (const float *)cache, cap, width, kofs, B);
  return hipGetLastError();
}

hipError_t launch_copy_rows(int dtype, void *dst, int64_t ldd, const void *src, int64_t lds,
                            int64_t rows, int width, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t es = dtype == BF16 ? 2 : 4;
  if ((width * es) % 16 == 0 && (ldd * es) % 16 == 0 && (lds * es) % 16 == 0 &&
      ((uintptr_t)dst & 15) == 0 && ((uintptr_t)src & 15) == 0) {
    const int nch = (int)(width * es / 16);
    const int64_t total = rows * nch;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(copy_rows16_kernel, dim3(blocks), dim3(256), 0, st, (uint4 *)dst, ldd * es / 16,
                       (const uint4 *)src, lds * es / 16, rows, nch);
    return hipGetLastError();
  }
  int64_t total = rows * width;
  unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  if (dtype == BF16)
    hipLaunchKernelGGL(copy_rows_kernel<bf16>, dim3(blocks), dim3(256), 0, st, (bf16 *)dst, ldd,
                       (const bf16 *)src, lds, rows, width);
  else
    hipLaunchKernelGGL(copy_rows_kernel<float>, dim3(blocks), dim3(256), 0, st, (float *)dst,
                       ldd, (const float *)src, lds, rows, width);
  return hipGetLastError();
}

hipError_t launch_cache_append(int dtype, void *cache, int64_t cap, const int32_t *lens, int q_len,
                               const void *src, int64_t lds, int64_t batch, int width,
                               hipStream_t st) {
  if (batch <= 0 || q_len <= 0) return hipSuccess;
  const unsigned rows = (unsigned)(batch * q_len);
  if (dtype == BF16)
    hipLaunchKernelGGL(cache_append_kernel<bf16>, dim3(rows), dim3(256), 0, st, (bf16 *)cache, cap,
                       lens, q_len, (const bf16 *)src, lds, width);
  else
    hipLaunchKernelGGL(cache_append_kernel<float>, dim3(rows), dim3(256), 0, st, (float *)cache,
                       cap, lens, q_len, (const float *)src, lds, width);
  return hipGetLastError();
}

hipError_t launch_decode_positions(const int32_t *lens, int batch, int q_len, int32_t *pos,
                                   hipStream_t st) {
  const int n = batch * q_len;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     lens, n, q_len, pos);
  return hipGetLastError();
}

}  // namespace mla
