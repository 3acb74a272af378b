// MFMA GEMM C = A B^T for the MLA projections (gfx950).
//
// A is [M, K] with K contiguous; B is [N, K] with K contiguous (nn.Linear
// weights, y = x W^T) or, for the per-head query absorption, [K, N] with N
// contiguous.  fp32 accumulation; bf16 uses v_mfma_f32_32x32x16_bf16 and
// fp32 uses v_mfma_f32_32x32x2_f32.  The epilogue scatters columns to
// per-head tensors (see GemmSeg), so the projections write the head-major
// layouts the attention kernels read without extra passes.
//
// Tiling: 128x128 output tile per 256-thread workgroup, four waves in a 2x2
// grid of 64x64 wave tiles (2x2 MFMA tiles each), K in 64-byte slabs staged
// through double-buffered LDS with register prefetch of the next slab.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int BM = 128, BN = 128;

struct GemmParams {
  const void *A;
  int64_t lda, strideA, strideB, strideC;
  int M, N, K, S, H, nseg;
  GemmSeg seg[3];
};

template <typename T> struct GemmCfg {
  static constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte chunk
  static constexpr int BK = 64 / sizeof(T);    // elements per K slab
  static constexpr int PITCH = BK + VEC;       // LDS row pitch (elements)
};

template <typename T>
__device__ inline void load_chunk(const T *p, bool ok, uint4 &v) {
  if (ok) v = *reinterpret_cast<const uint4 *>(p);
  else v = make_uint4(0, 0, 0, 0);
}

template <typename T, bool BKN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  using C = GemmCfg<T>;
  using MF = Mfma32<T>;
  constexpr int BK = C::BK, PITCH = C::PITCH, VEC = C::VEC;
  __shared__ __attribute__((aligned(16))) T As[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) T Bs[2][BN * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.z;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const T *A = reinterpret_cast<const T *>(p.A) + (int64_t)z * p.strideA;

  // global -> register staging: each thread owns two 16-byte chunks of A and B
  uint4 ra[2], rb[2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = tid + 256 * i;
      int row = c >> 2, ch = c & 3;
      int m = m0 + row, k = k0 + ch * VEC;
      load_chunk<T>(A + (int64_t)m * p.lda + k, m < p.M && k < p.K, ra[i]);
    }
    if constexpr (!BKN) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int row = c >> 2, ch = c & 3;
        int n = n0 + row, k = k0 + ch * VEC;
        int s = (p.nseg > 1 && n >= p.seg[1].n_begin) ? ((p.nseg > 2 && n >= p.seg[2].n_begin) ? 2 : 1) : 0;
        const T *B = reinterpret_cast<const T *>(p.seg[s].B) + (int64_t)z * p.strideB;
        load_chunk<T>(B + (int64_t)(n - p.seg[s].n_begin) * p.seg[s].ldb + k,
                      n < p.N && k < p.K, rb[i]);
      }
    } else {
      constexpr int CPR = BN / VEC;  // chunks per k row of the tile
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int kr = c / CPR, nc = c % CPR;
        int k = k0 + kr, n = n0 + nc * VEC;
        const T *B = reinterpret_cast<const T *>(p.seg[0].B) + (int64_t)z * p.strideB;
        load_chunk<T>(B + (int64_t)k * p.seg[0].ldb + n, k < p.K && n < p.N, rb[i]);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = tid + 256 * i;
      int row = c >> 2, ch = c & 3;
      *reinterpret_cast<uint4 *>(&As[buf][row * PITCH + ch * VEC]) = ra[i];
    }
    if constexpr (!BKN) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int row = c >> 2, ch = c & 3;
        *reinterpret_cast<uint4 *>(&Bs[buf][row * PITCH + ch * VEC]) = rb[i];
      }
    } else {
      constexpr int CPR = BN / VEC;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int kr = c / CPR, nc = c % CPR;
        const T *v = reinterpret_cast<const T *>(&rb[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) Bs[buf][(nc * VEC + e) * PITCH + kr] = v[e];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (p.K + BK - 1) / BK;
  fetch(0);
  stash(0);
  __syncthreads();
  const int g = lane >> 5, l32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += MF::KSTEP) {
      typename MF::frag a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const typename MF::frag *>(
            &As[buf][(wm * 64 + i * 32 + l32) * PITCH + kk + g * MF::KPL]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const typename MF::frag *>(
            &Bs[buf][(wn * 64 + j * 32 + l32) * PITCH + kk + g * MF::KPL]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MF::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  // epilogue: scatter to the column range's destination
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    if (n >= p.N) continue;
    const int s = (p.nseg > 1 && n >= p.seg[1].n_begin) ? ((p.nseg > 2 && n >= p.seg[2].n_begin) ? 2 : 1) : 0;
    const GemmSeg &sg = p.seg[s];
    const int nn = n - sg.n_begin;
    const int h = nn / sg.dh, d = nn - h * sg.dh;
    T *Cb = reinterpret_cast<T *>(sg.C) + (int64_t)z * p.strideC + sg.off + d;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (m < p.M) {
          const int b = m / p.S, sq = m - b * p.S;
          Cb[((int64_t)(b * p.H + h) * p.S + sq) * sg.ld] = from_f32<T>(acc[i][j][r]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const GemmDesc &d, hipStream_t st) {
  if (d.M <= 0 || d.N <= 0 || d.K <= 0 || d.batch <= 0) return hipSuccess;
  GemmParams p;
  p.A = d.A;
  p.lda = d.lda;
  p.strideA = d.strideA;
  p.strideB = d.strideB;
  p.strideC = d.strideC;
  p.M = d.M;
  p.N = d.N;
  p.K = d.K;
  p.S = d.S;
  p.H = d.H;
  p.nseg = d.nseg;
  for (int i = 0; i < 3; ++i) p.seg[i] = d.seg[i];
  dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM, d.batch);
  dim3 block(256);
  if (d.dtype == BF16) {
    if (d.b_kn) hipLaunchKernelGGL((gemm_kernel<bf16, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<bf16, false>), grid, block, 0, st, p);
  } else {
    if (d.b_kn) hipLaunchKernelGGL((gemm_kernel<float, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<float, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mla
