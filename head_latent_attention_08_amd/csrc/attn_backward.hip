// Causal attention backward (dQ, dK, dV) for gfx950: the gradients of the
// per-head forward of "The Evolving Transformer -- DeepSeek V2 & V3",
// section 01 (P = softmax(scale Q K^T, causal tril mask), O = P V):
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three passes, each a wave per row, vector-ALU arithmetic in fp32:
//  1. per query row i: lse_i = log sum_j<=i exp(s_ij) and delta_i =
//     rowsum(dO_i * O_i), into a workspace of 8 bytes per row;
//  2. per key row j: over the queries i >= j, 64 at a time (a lane per
//     query: s_ij, p_ij = exp(s_ij - lse_i), dp_ij, ds_ij), then the wave
//     turns to channels (a lane per channel) and accumulates
//     dV_j += p_ij dO_i and dK_j += ds_ij Q_i, reading the 64 rows coalesced;
//  3. per query row i: the same over keys j <= i for dQ_i += ds_ij K_j.
// P is recomputed from lse, never stored.  Rows are [BH, S, d] contiguous,
// d a multiple of 8 and at most 256, pointers 16-byte aligned.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int AB_DMAX = 256;

template <typename T> __device__ inline void ab_load8(const T *p, float *f) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const bf16 *h = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
  } else {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// dot of a global row (n elements) with an LDS vector
template <typename T> __device__ inline float ab_dot(const T *row, const float *v, int n) {
  float s = 0.f;
  for (int c = 0; c < n; c += 8) {
    float f[8];
    ab_load8(row + c, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(f[e], v[c + e], s);
  }
  return s;
}

__device__ inline float ab_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T> __device__ inline float ab_ld(const T *p) { return (float)*p; }

// pass 1: lse and delta of query row (bh, i)
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_rowstats_kernel(AttnBwdArgs a) {
  __shared__ float qs[4][AB_DMAX];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= (int64_t)a.BH * a.S) return;
  const int i = (int)(row % a.S);
  const int64_t bh = row / a.S;
  const T *q = reinterpret_cast<const T *>(a.q) + row * a.dqk;
  const T *kb = reinterpret_cast<const T *>(a.k) + bh * a.S * a.dqk;
  for (int c = lane; c < a.dqk; c += 64) qs[wv][c] = ab_ld(q + c);
  const T *o = reinterpret_cast<const T *>(a.o) + row * a.dv;
  const T *dO = reinterpret_cast<const T *>(a.dout) + row * a.dv;
  float d = 0.f;
  for (int c = lane; c < a.dv; c += 64) d = fmaf(ab_ld(o + c), ab_ld(dO + c), d);
  d = ab_wave_sum(d);
  __builtin_amdgcn_wave_barrier();
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 <= i; j0 += 64) {
    const int j = j0 + lane;
    if (j <= i) {
      const float s = a.scale * ab_dot(kb + (int64_t)j * a.dqk, qs[wv], a.dqk);
      const float mn = fmaxf(m, s);
      l = l * expf(m - mn) + expf(s - mn);
      m = mn;
    }
  }
  float M = m;
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) M = fmaxf(M, __shfl_xor(M, o2));
  const float L = ab_wave_sum(m == -INFINITY ? 0.f : l * expf(m - M));
  if (lane == 0) {
    a.lse[row] = M + logf(L);
    a.delta[row] = d;
  }
}

// pass 2: dK and dV of key row (bh, j)
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  __shared__ float ks[4][AB_DMAX], vs[4][AB_DMAX], ps[4][64], dss[4][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= (int64_t)a.BH * a.S) return;
  const int j = (int)(row % a.S);
  const int64_t bh = row / a.S;
  const T *qb = reinterpret_cast<const T *>(a.q) + bh * a.S * a.dqk;
  const T *db = reinterpret_cast<const T *>(a.dout) + bh * a.S * a.dv;
  const float *lse = a.lse + bh * a.S, *delta = a.delta + bh * a.S;
  for (int c = lane; c < a.dqk; c += 64) ks[wv][c] = ab_ld(reinterpret_cast<const T *>(a.k) + row * a.dqk + c);
  for (int c = lane; c < a.dv; c += 64) vs[wv][c] = ab_ld(reinterpret_cast<const T *>(a.v) + row * a.dv + c);
  __builtin_amdgcn_wave_barrier();
  float dk[AB_DMAX / 64] = {0.f, 0.f, 0.f, 0.f}, dv[AB_DMAX / 64] = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = j; i0 < a.S; i0 += 64) {
    const int i = i0 + lane;
    float p = 0.f, ds = 0.f;
    if (i < a.S) {
      const float s = a.scale * ab_dot(qb + (int64_t)i * a.dqk, ks[wv], a.dqk);
      p = expf(s - lse[i]);
      const float dp = ab_dot(db + (int64_t)i * a.dv, vs[wv], a.dv);
      ds = p * (dp - delta[i]);
    }
    ps[wv][lane] = p;
    dss[wv][lane] = ds;
    __builtin_amdgcn_wave_barrier();
    const int n = min(64, a.S - i0);
    for (int t = 0; t < n; ++t) {
      const float pt = ps[wv][t], dt = dss[wv][t];
      const T *qr = qb + (int64_t)(i0 + t) * a.dqk, *dr = db + (int64_t)(i0 + t) * a.dv;
#pragma unroll
      for (int u = 0; u < AB_DMAX / 64; ++u) {
        const int c = lane + 64 * u;
        if (c < a.dqk) dk[u] = fmaf(dt, ab_ld(qr + c), dk[u]);
        if (c < a.dv) dv[u] = fmaf(pt, ab_ld(dr + c), dv[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  T *dkr = reinterpret_cast<T *>(a.dk) + row * a.dqk;
  T *dvr = reinterpret_cast<T *>(a.dvo) + row * a.dv;
#pragma unroll
  for (int u = 0; u < AB_DMAX / 64; ++u) {
    const int c = lane + 64 * u;
    if (c < a.dqk) dkr[c] = (T)(a.scale * dk[u]);
    if (c < a.dv) dvr[c] = (T)dv[u];
  }
}

// pass 3: dQ of query row (bh, i)
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  __shared__ float qs[4][AB_DMAX], dos[4][AB_DMAX], dss[4][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= (int64_t)a.BH * a.S) return;
  const int i = (int)(row % a.S);
  const int64_t bh = row / a.S;
  const T *kb = reinterpret_cast<const T *>(a.k) + bh * a.S * a.dqk;
  const T *vb = reinterpret_cast<const T *>(a.v) + bh * a.S * a.dv;
  for (int c = lane; c < a.dqk; c += 64) qs[wv][c] = ab_ld(reinterpret_cast<const T *>(a.q) + row * a.dqk + c);
  for (int c = lane; c < a.dv; c += 64) dos[wv][c] = ab_ld(reinterpret_cast<const T *>(a.dout) + row * a.dv + c);
  const float lse = a.lse[row], delta = a.delta[row];
  __builtin_amdgcn_wave_barrier();
  float dq[AB_DMAX / 64] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 <= i; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j <= i) {
      const float s = a.scale * ab_dot(kb + (int64_t)j * a.dqk, qs[wv], a.dqk);
      const float p = expf(s - lse);
      const float dp = ab_dot(vb + (int64_t)j * a.dv, dos[wv], a.dv);
      ds = p * (dp - delta);
    }
    dss[wv][lane] = ds;
    __builtin_amdgcn_wave_barrier();
    const int n = min(64, i + 1 - j0);
    for (int t = 0; t < n; ++t) {
      const float dt = dss[wv][t];
      const T *kr = kb + (int64_t)(j0 + t) * a.dqk;
#pragma unroll
      for (int u = 0; u < AB_DMAX / 64; ++u) {
        const int c = lane + 64 * u;
        if (c < a.dqk) dq[u] = fmaf(dt, ab_ld(kr + c), dq[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  T *dqr = reinterpret_cast<T *>(a.dq) + row * a.dqk;
#pragma unroll
  for (int u = 0; u < AB_DMAX / 64; ++u) {
    const int c = lane + 64 * u;
    if (c < a.dqk) dqr[c] = (T)(a.scale * dq[u]);
  }
}

template <typename T> hipError_t launch_t(const AttnBwdArgs &a, hipStream_t st) {
  const int64_t rows = (int64_t)a.BH * a.S;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipLaunchKernelGGL(attn_bwd_rowstats_kernel<T>, grid, block, 0, st, a);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<T>, grid, block, 0, st, a);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<T>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_backward(int dtype, const AttnBwdArgs &a, hipStream_t st) {
  if ((int64_t)a.BH * a.S == 0) return hipSuccess;
  return dtype == BF16 ? launch_t<bf16>(a, st) : launch_t<float>(a, st);
}

}  // namespace mla
