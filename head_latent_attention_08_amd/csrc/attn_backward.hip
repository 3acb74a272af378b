// Causal attention backward (dQ, dK, dV) for gfx950: the gradients of the
// per-head forward of "The Evolving Transformer -- DeepSeek V2 & V3",
// section 01 (P = softmax(scale Q K^T, causal tril mask), O = P V):
//
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three passes, each a wave per 4 rows of a head, vector-ALU arithmetic in fp32:
//  1. per 4 query rows i: lse_i = log sum_j<=i exp(s_ij) and delta_i =
//     rowsum(dO_i * O_i), into a workspace of 8 bytes per row;
//  2. per 4 key rows j: over the queries i >= j, 64 at a time (a lane per
//     query: s_ij, p_ij = exp(s_ij - lse_i), dp_ij, ds_ij for the 4 keys),
//     then the wave turns to channels (a lane per channel) and accumulates
//     dV_j += p_ij dO_i and dK_j += ds_ij Q_i, reading the 64 rows coalesced
//     once for the 4 keys;
//  3. per 4 query rows i: the same over keys j <= i for dQ_i += ds_ij K_j.
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

// R rows of a head per wave in passes 2 and 3: each streamed row is read
// once for all R of them (loads shared across R dot products and R sets of
// accumulators).
constexpr int AB_R = 4;

// dot of one global row with R LDS vectors
template <typename T>
__device__ inline void ab_dot_r(const T *row, const float (*v)[AB_DMAX], int n, float *out) {
#pragma unroll
  for (int r = 0; r < AB_R; ++r) out[r] = 0.f;
  for (int c = 0; c < n; c += 8) {
    float f[8];
    ab_load8(row + c, f);
#pragma unroll
    for (int r = 0; r < AB_R; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) out[r] = fmaf(f[e], v[r][c + e], out[r]);
  }
}

// pass 1: lse and delta of query rows i0 .. i0 + R - 1 of head bh
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_rowstats_kernel(AttnBwdArgs a) {
  __shared__ float qs[4][AB_R][AB_DMAX];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nb = (a.S + AB_R - 1) / AB_R;
  const int64_t w = (int64_t)blockIdx.x * 4 + wv;
  if (w >= (int64_t)a.BH * nb) return;
  const int64_t bh = w / nb;
  const int i0 = (int)(w - bh * nb) * AB_R;
  const int nq = min(AB_R, a.S - i0);
  const T *kb = reinterpret_cast<const T *>(a.k) + bh * a.S * a.dqk;
  float d[AB_R];
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    const bool ok = r < nq;
    const int64_t row = bh * a.S + i0 + r;
    for (int c = lane; c < a.dqk; c += 64)
      qs[wv][r][c] = ok ? ab_ld(reinterpret_cast<const T *>(a.q) + row * a.dqk + c) : 0.f;
    float x = 0.f;
    if (ok)
      for (int c = lane; c < a.dv; c += 64)
        x = fmaf(ab_ld(reinterpret_cast<const T *>(a.o) + row * a.dv + c),
                 ab_ld(reinterpret_cast<const T *>(a.dout) + row * a.dv + c), x);
    d[r] = ab_wave_sum(x);
  }
  __builtin_amdgcn_wave_barrier();
  float m[AB_R], l[AB_R];
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
  const int last = i0 + nq - 1;
  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + lane;
    if (j <= last) {
      float s[AB_R];
      ab_dot_r(kb + (int64_t)j * a.dqk, qs[wv], a.dqk, s);
#pragma unroll
      for (int r = 0; r < AB_R; ++r) {
        if (r < nq && j <= i0 + r) {
          const float x = a.scale * s[r];
          const float mn = fmaxf(m[r], x);
          l[r] = l[r] * expf(m[r] - mn) + expf(x - mn);
          m[r] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    float M = m[r];
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) M = fmaxf(M, __shfl_xor(M, o2));
    const float L = ab_wave_sum(m[r] == -INFINITY ? 0.f : l[r] * expf(m[r] - M));
    if (lane == 0 && r < nq) {
      a.lse[bh * a.S + i0 + r] = M + logf(L);
      a.delta[bh * a.S + i0 + r] = d[r];
    }
  }
}

// pass 2: dK and dV of key rows j0 .. j0 + R - 1 of head bh
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  __shared__ float ks[4][AB_R][AB_DMAX], vs[4][AB_R][AB_DMAX], ps[4][AB_R][64], dss[4][AB_R][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nb = (a.S + AB_R - 1) / AB_R;
  const int64_t w = (int64_t)blockIdx.x * 4 + wv;
  if (w >= (int64_t)a.BH * nb) return;
  const int64_t bh = w / nb;
  const int j0 = (int)(w - bh * nb) * AB_R;
  const T *qb = reinterpret_cast<const T *>(a.q) + bh * a.S * a.dqk;
  const T *db = reinterpret_cast<const T *>(a.dout) + bh * a.S * a.dv;
  const float *lse = a.lse + bh * a.S, *delta = a.delta + bh * a.S;
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    const bool ok = j0 + r < a.S;
    const int64_t row = bh * a.S + j0 + r;
    for (int c = lane; c < a.dqk; c += 64)
      ks[wv][r][c] = ok ? ab_ld(reinterpret_cast<const T *>(a.k) + row * a.dqk + c) : 0.f;
    for (int c = lane; c < a.dv; c += 64)
      vs[wv][r][c] = ok ? ab_ld(reinterpret_cast<const T *>(a.v) + row * a.dv + c) : 0.f;
  }
  __builtin_amdgcn_wave_barrier();
  float dk[AB_R][AB_DMAX / 64], dv[AB_R][AB_DMAX / 64];
#pragma unroll
  for (int r = 0; r < AB_R; ++r)
#pragma unroll
    for (int u = 0; u < AB_DMAX / 64; ++u) dk[r][u] = dv[r][u] = 0.f;
  for (int i0 = j0; i0 < a.S; i0 += 64) {
    const int i = i0 + lane;
    float s[AB_R], dp[AB_R];
    if (i < a.S) {
      ab_dot_r(qb + (int64_t)i * a.dqk, ks[wv], a.dqk, s);
      ab_dot_r(db + (int64_t)i * a.dv, vs[wv], a.dv, dp);
    }
#pragma unroll
    for (int r = 0; r < AB_R; ++r) {
      float p = 0.f, ds = 0.f;
      if (i < a.S && j0 + r <= i) {   // key j0 + r is visible to query i (and inside the sequence)
        p = expf(a.scale * s[r] - lse[i]);
        ds = p * (dp[r] - delta[i]);
      }
      ps[wv][r][lane] = p;
      dss[wv][r][lane] = ds;
    }
    __builtin_amdgcn_wave_barrier();
    const int n = min(64, a.S - i0);
    for (int t = 0; t < n; ++t) {
      const T *qr = qb + (int64_t)(i0 + t) * a.dqk, *dr = db + (int64_t)(i0 + t) * a.dv;
#pragma unroll
      for (int u = 0; u < AB_DMAX / 64; ++u) {
        const int c = lane + 64 * u;
        const float qv = c < a.dqk ? ab_ld(qr + c) : 0.f;
        const float gv = c < a.dv ? ab_ld(dr + c) : 0.f;
#pragma unroll
        for (int r = 0; r < AB_R; ++r) {
          dk[r][u] = fmaf(dss[wv][r][t], qv, dk[r][u]);
          dv[r][u] = fmaf(ps[wv][r][t], gv, dv[r][u]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    if (j0 + r >= a.S) break;
    const int64_t row = bh * a.S + j0 + r;
    T *dkr = reinterpret_cast<T *>(a.dk) + row * a.dqk;
    T *dvr = reinterpret_cast<T *>(a.dvo) + row * a.dv;
#pragma unroll
    for (int u = 0; u < AB_DMAX / 64; ++u) {
      const int c = lane + 64 * u;
      if (c < a.dqk) dkr[c] = (T)(a.scale * dk[r][u]);
      if (c < a.dv) dvr[c] = (T)dv[r][u];
    }
  }
}

// pass 3: dQ of query rows i0 .. i0 + R - 1 of head bh
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  __shared__ float qs[4][AB_R][AB_DMAX], dos[4][AB_R][AB_DMAX], dss[4][AB_R][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nb = (a.S + AB_R - 1) / AB_R;
  const int64_t w = (int64_t)blockIdx.x * 4 + wv;
  if (w >= (int64_t)a.BH * nb) return;
  const int64_t bh = w / nb;
  const int i0 = (int)(w - bh * nb) * AB_R;
  const int nq = min(AB_R, a.S - i0);
  const T *kb = reinterpret_cast<const T *>(a.k) + bh * a.S * a.dqk;
  const T *vb = reinterpret_cast<const T *>(a.v) + bh * a.S * a.dv;
  float lse[AB_R], delta[AB_R];
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    const bool ok = r < nq;
    const int64_t row = bh * a.S + i0 + r;
    for (int c = lane; c < a.dqk; c += 64)
      qs[wv][r][c] = ok ? ab_ld(reinterpret_cast<const T *>(a.q) + row * a.dqk + c) : 0.f;
    for (int c = lane; c < a.dv; c += 64)
      dos[wv][r][c] = ok ? ab_ld(reinterpret_cast<const T *>(a.dout) + row * a.dv + c) : 0.f;
    lse[r] = ok ? a.lse[row] : 0.f;
    delta[r] = ok ? a.delta[row] : 0.f;
  }
  __builtin_amdgcn_wave_barrier();
  float dq[AB_R][AB_DMAX / 64];
#pragma unroll
  for (int r = 0; r < AB_R; ++r)
#pragma unroll
    for (int u = 0; u < AB_DMAX / 64; ++u) dq[r][u] = 0.f;
  const int last = i0 + nq - 1;  // the last query row of the wave
  for (int j0 = 0; j0 <= last; j0 += 64) {
    const int j = j0 + lane;
    float s[AB_R], dp[AB_R];
    if (j <= last) {
      ab_dot_r(kb + (int64_t)j * a.dqk, qs[wv], a.dqk, s);
      ab_dot_r(vb + (int64_t)j * a.dv, dos[wv], a.dv, dp);
    }
#pragma unroll
    for (int r = 0; r < AB_R; ++r) {
      float ds = 0.f;
      if (r < nq && j <= i0 + r) {
        const float p = expf(a.scale * s[r] - lse[r]);
        ds = p * (dp[r] - delta[r]);
      }
      dss[wv][r][lane] = ds;
    }
    __builtin_amdgcn_wave_barrier();
    const int n = min(64, last + 1 - j0);
    for (int t = 0; t < n; ++t) {
      const T *kr = kb + (int64_t)(j0 + t) * a.dqk;
#pragma unroll
      for (int u = 0; u < AB_DMAX / 64; ++u) {
        const int c = lane + 64 * u;
        const float kv = c < a.dqk ? ab_ld(kr + c) : 0.f;
#pragma unroll
        for (int r = 0; r < AB_R; ++r) dq[r][u] = fmaf(dss[wv][r][t], kv, dq[r][u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int r = 0; r < AB_R; ++r) {
    if (r >= nq) break;
    T *dqr = reinterpret_cast<T *>(a.dq) + (bh * a.S + i0 + r) * a.dqk;
#pragma unroll
    for (int u = 0; u < AB_DMAX / 64; ++u) {
      const int c = lane + 64 * u;
      if (c < a.dqk) dqr[c] = (T)(a.scale * dq[r][u]);
    }
  }
}

// RMSNorm backward of y = x r g, r = (mean(x^2) + eps)^-1/2 per row:
// dx = r (g dy) - x r^3 mean(x g dy), one workgroup per row (rinv kept per
// row).  dg[c] = sum over rows of dy x r in two fixed-order levels: chunks of
// RB_CHUNK rows give fp32 partials (one thread per column of a chunk), then
// the partials of each column are added chunk by chunk (deterministic, and
// the whole GPU takes part instead of one workgroup per 256 columns).
constexpr int RB_CHUNK = 64;

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_rows_kernel(const T *x, int64_t ldx, const T *dy, int64_t ldy,
                                                               const T *g, int n, float eps, T *dx, int64_t lddx,
                                                               float *rinv) {
  __shared__ float red[2][4];
  const int64_t row = blockIdx.x;
  const T *xr = x + row * ldx, *dr = dy + row * ldy;
  float ss = 0.f, xg = 0.f;
  for (int c = threadIdx.x; c < n; c += 256) {
    const float xv = (float)xr[c];
    ss = fmaf(xv, xv, ss);
    xg = fmaf(xv, (float)g[c] * (float)dr[c], xg);
  }
  ss = ab_wave_sum(ss);
  xg = ab_wave_sum(xg);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = ss;
    red[1][threadIdx.x >> 6] = xg;
  }
  __syncthreads();
  ss = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  xg = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float r = 1.f / sqrtf(ss / n + eps);
  const float k = r * r * r * xg / n;
  for (int c = threadIdx.x; c < n; c += 256)
    dx[row * lddx + c] = (T)(r * (float)g[c] * (float)dr[c] - (float)xr[c] * k);
  if (threadIdx.x == 0) rinv[row] = r;
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_dg_part_kernel(const T *x, int64_t ldx, const T *dy,
                                                                  int64_t ldy, int64_t rows, int n,
                                                                  const float *rinv, float *part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * RB_CHUNK;
  if (c >= n) return;
  const int64_t r1 = min(r0 + RB_CHUNK, rows);
  float acc = 0.f;
  for (int64_t r = r0; r < r1; ++r) acc = fmaf((float)dy[r * ldy + c] * (float)x[r * ldx + c], rinv[r], acc);
  part[(int64_t)blockIdx.y * n + c] = acc;
}

__global__ __launch_bounds__(256) void rmsnorm_bwd_dg_sum_kernel(const float *part, int chunks, int n, float *dg) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  float acc = 0.f;
  for (int i = 0; i < chunks; ++i) acc += part[(int64_t)i * n + c];
  dg[c] = acc;
}

template <typename T>
hipError_t launch_rms_t(const void *x, int64_t ldx, const void *dy, int64_t ldy, const void *g, int64_t rows, int n,
                        float eps, void *dx, int64_t lddx, float *dg, float *scratch, hipStream_t st) {
  float *rinv = scratch, *part = scratch + rows;
  const int chunks = (int)((rows + RB_CHUNK - 1) / RB_CHUNK);
  hipLaunchKernelGGL(rmsnorm_bwd_rows_kernel<T>, dim3((unsigned)rows), dim3(256), 0, st,
                     reinterpret_cast<const T *>(x), ldx, reinterpret_cast<const T *>(dy), ldy,
                     reinterpret_cast<const T *>(g), n, eps, reinterpret_cast<T *>(dx), lddx, rinv);
  hipLaunchKernelGGL(rmsnorm_bwd_dg_part_kernel<T>, dim3((unsigned)((n + 255) / 256), (unsigned)chunks), dim3(256), 0,
                     st, reinterpret_cast<const T *>(x), ldx, reinterpret_cast<const T *>(dy), ldy, rows, n, rinv,
                     part);
  hipLaunchKernelGGL(rmsnorm_bwd_dg_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, chunks,
                     n, dg);
  return hipGetLastError();
}

template <typename T> hipError_t launch_t(const AttnBwdArgs &a, hipStream_t st) {
  const dim3 block(256);
  const int64_t blocks = (int64_t)a.BH * ((a.S + AB_R - 1) / AB_R);
  const dim3 rgrid((unsigned)((blocks + 3) / 4));
  hipLaunchKernelGGL(attn_bwd_rowstats_kernel<T>, rgrid, block, 0, st, a);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<T>, rgrid, block, 0, st, a);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<T>, rgrid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

size_t rmsnorm_backward_scratch_floats(int64_t rows, int n) {
  return (size_t)rows + (size_t)((rows + RB_CHUNK - 1) / RB_CHUNK) * (size_t)n;
}

hipError_t launch_rmsnorm_backward(int dtype, const void *x, int64_t ldx, const void *dy, int64_t ldy, const void *g,
                                   int64_t rows, int n, float eps, void *dx, int64_t lddx, float *dg, float *scratch,
                                   hipStream_t st) {
  if (rows == 0) return hipSuccess;
  return dtype == BF16 ? launch_rms_t<bf16>(x, ldx, dy, ldy, g, rows, n, eps, dx, lddx, dg, scratch, st)
                       : launch_rms_t<float>(x, ldx, dy, ldy, g, rows, n, eps, dx, lddx, dg, scratch, st);
}

hipError_t launch_attention_backward(int dtype, const AttnBwdArgs &a, hipStream_t st) {
  if ((int64_t)a.BH * a.S == 0) return hipSuccess;
  if (attention_backward_mfma_supported(dtype, a.dqk, a.dv)) return launch_attention_backward_mfma(a, st);
  return dtype == BF16 ? launch_t<bf16>(a, st) : launch_t<float>(a, st);
}

}  // namespace mla
