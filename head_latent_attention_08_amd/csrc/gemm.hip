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

#include <numeric>

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
  // row RMSNorm split over a producer / consumer pair (GemmDesc)
  float *rn_part;
  const bf16 *rn_gain;
  int rn_cols;
  const float *rs_part;
  int rs_chunks;
  float rs_eps;
  const float *rope_tab;
  int rope_seg, rope_conv;
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

template <typename T, bool BKN, bool AKM>
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
    if constexpr (!AKM) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int row = c >> 2, ch = c & 3;
        int m = m0 + row, k = k0 + ch * VEC;
        load_chunk<T>(A + (int64_t)m * p.lda + k, m < p.M && k < p.K, ra[i]);
      }
    } else {
      // A stored [K][M] (M contiguous): chunks of VEC consecutive m of one k
      constexpr int CPR = BM / VEC;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int kr = c / CPR, mc = c % CPR;
        int k = k0 + kr, m = m0 + mc * VEC;
        load_chunk<T>(A + (int64_t)k * p.lda + m, k < p.K && m < p.M, ra[i]);
      }
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
    if constexpr (!AKM) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int row = c >> 2, ch = c & 3;
        *reinterpret_cast<uint4 *>(&As[buf][row * PITCH + ch * VEC]) = ra[i];
      }
    } else {
      constexpr int CPR = BM / VEC;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int c = tid + 256 * i;
        int kr = c / CPR, mc = c % CPR;
        const T *v = reinterpret_cast<const T *>(&ra[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) As[buf][(mc * VEC + e) * PITCH + kr] = v[e];
      }
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
    T *Cb = reinterpret_cast<T *>(sg.C) + (int64_t)z * p.strideC;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (m < p.M) {
          const int b = m / p.S, sq = m - b * p.S;
          const int64_t at = sg.tr ? ((int64_t)(b * p.H + h) * sg.dh + d) * p.S + sq
                                   : ((int64_t)(b * p.H + h) * p.S + sq) * sg.ld + sg.off + d;
          Cb[at] = from_f32<T>(acc[i][j][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel for the prefill projections (M in the thousands).
//
// A (64*TM) x (64*TN) output tile per 256-thread workgroup: four waves in a
// 2x2 grid of (32*TM) x (32*TN) wave tiles (TM x TN MFMA 32x32 tiles, up to
// 256 fp32 accumulators per lane held in the accumulation registers), one
// wave per SIMD; the projections use the square 256x256 tile (TM = TN = 4),
// short-K ones 256x128 (TM = 4, TN = 2: 128 accumulators, two waves per
// SIMD, three stages).
// A copy block of B rows takes its column range's weight matrix, so range
// starts only need to be multiples of 16 (channel-major ranges, whose stores
// differ, start on tile boundaries).
//
// K advances in 32-wide slabs through four LDS stages.  LDS rows are 32
// elements (four 16-byte chunks) with chunk j of row r stored at position
// j ^ ((r / 4) % 4), so the sixteen consecutive rows one quarter wave reads
// for a fragment fall in distinct banks.
//
// Tiles are numbered so that each of the eight XCDs (which take workgroup ids
// round-robin) works on a contiguous run of tiles, walked in groups of
// group_m tile rows, so concurrently running tiles share A and B slabs in that
// XCD's L2 (taller groups pay off for long K, flat ones for short K, where
// the output stores dominate).
//
// The accumulators leave through LDS: the tile is written there as bf16, then
// every thread stores 16-byte runs of 8 consecutive columns, which fall in one
// head of one column range of the destination (all column ranges and head
// widths are multiples of 8), so the head-scatter store stays vectorised.
constexpr int GB_K = 32, GB_THREADS = 256;
constexpr int GB_STAGES = 4;

template <int TM, int TN, int NST> struct BigTile {
  static constexpr int M = 64 * TM, N = 64 * TN;            // output tile
  static constexpr int CPITCH = N + 8;                      // epilogue LDS pitch (elements)
  static constexpr int STAGE = (M + N) * GB_K;              // elements per operand stage
  static constexpr int LDS = M * CPITCH > NST * STAGE ? M * CPITCH : NST * STAGE;
  static constexpr int ABLK = M / 16, NQ = (M + N) / 64;    // A copy blocks; copies per wave per slab
  static constexpr int QH = (NQ + 1) / 2;                   // copies spread over the first k-step
  static_assert(ABLK % 4 == 0 && (M + N) % 64 == 0, "copy blocks must split evenly over four waves");
};

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left open (gfx9 encoding)
constexpr int GB_VMCNT0 = (7 << 4) | (15 << 8);
// at most n vector-memory operations of this wave outstanding
#define GB_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// LDS position of element (r, k) of a 32-wide operand slab: 64-byte rows whose
// four 16-byte chunks are XOR-permuted by (r / 4) % 4, so the 16 consecutive
// rows one fragment read of a quarter wave touches fall in distinct banks.
__device__ inline int swz(int r, int k) { return r * GB_K + ((((k >> 3) ^ (r >> 2)) & 3) << 3) + (k & 7); }

__device__ inline int seg_of(const GemmParams &p, int n) {
  return (p.nseg > 1 && n >= p.seg[1].n_begin) ? ((p.nseg > 2 && n >= p.seg[2].n_begin) ? 2 : 1) : 0;
}

// Fields of column range s, read with constant indices only (a dynamic index
// into the kernel-argument struct would copy it to scratch memory).
#define SEG_FIELD(p, s, f) ((s) == 0 ? (p).seg[0].f : ((s) == 1 ? (p).seg[1].f : (p).seg[2].f))

// A pointer the whole wave holds, moved to scalar registers (inline-asm
// scalar operands need it there even when the compiler computed it with
// vector instructions).
template <typename P> __device__ inline P *uniform_ptr(P *q) {
  const uint64_t v = (uint64_t)q;
  return reinterpret_cast<P *>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                               (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}

// Row-major stores of one thread's 8-column run: rows r0, r0 + RSTEP, .. of
// the LDS tile, U at a time (their LDS reads issued together).  dst points at
// row r0's destination; a step moves it RSTEP rows down its sequence, and a
// step past the sequence's end (s >= S) on to the next sequence, H - 1
// sequences of this head's rows further.  With GAIN the values are scaled by
// gv (bf16 products, as stored by a split-RMSNorm producer).
template <int PASSES, int U, int RSTEP, int CPITCH, bool GAIN>
__device__ __forceinline__ void store_row_runs(const bf16 *Cs, int r0, int cc, bf16 *dst, int64_t ld, int m, int M,
                                               int sq, int S, int64_t wrap, bf16x8 gv) {
  for (int it = 0; it < PASSES; it += U) {
    bf16x8 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const bf16x8 *>(&Cs[(r0 + RSTEP * (it + u)) * CPITCH + cc * 8]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (m < M) {
        if constexpr (GAIN) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[u][e] = (bf16)((float)v[u][e] * (float)gv[e]);
        }
        *reinterpret_cast<bf16x8 *>(dst) = v[u];
      }
      m += RSTEP;
      sq += RSTEP;
      dst += RSTEP * ld;
      while (sq >= S) {
        sq -= S;
        dst += wrap;
      }
    }
  }
}

// vmcnt immediates of the K loop, per wave: q copies per slab
template <int Q> __device__ inline void wait_slabs_outstanding(int slabs) {
  if (slabs >= 4) __builtin_amdgcn_s_waitcnt(GB_VMCNT(4 * Q));
  else if (slabs == 3) __builtin_amdgcn_s_waitcnt(GB_VMCNT(3 * Q));
  else if (slabs == 2) __builtin_amdgcn_s_waitcnt(GB_VMCNT(2 * Q));
  else if (slabs == 1) __builtin_amdgcn_s_waitcnt(GB_VMCNT(Q));
  else __builtin_amdgcn_s_waitcnt(GB_VMCNT0);
}

// Launch window: output columns [n_base, n_base + tiles_n * tile N) of every row.
template <int TM, int TN, int GB_NST>
__global__ __launch_bounds__(GB_THREADS) __attribute__((amdgpu_waves_per_eu(TM * TN <= 8 ? 2 : 1))) void gemm_big_kernel(GemmParams p, int tiles_m, int tiles_n,
                                                              int n_base, int remap, int group_m,
                                                              int cstride) {
  using BT = BigTile<TM, TN, GB_NST>;
  constexpr int NQ = BT::NQ, QH = BT::QH, ABLK = BT::ABLK;
  __shared__ __attribute__((aligned(16))) bf16 lds[BT::LDS];

  // tile index: contiguous run per XCD, then grouped row-major order
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (remap) t = (t & 7) * (T >> 3) + (t >> 3);
  const int per_group = group_m * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int tm = first_m + (t % per_group) % gm;
  const int tn = (t % per_group) / gm * cstride % tiles_n;  // cstride: coprime column stride (or 1)
  const int m0 = tm * BT::M, n0 = n_base + tn * BT::N;
  const int nk = p.K / GB_K;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds M0
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;
  const bf16 *A = reinterpret_cast<const bf16 *>(p.A);

  // Slabs of 32 k are copied from global memory straight into LDS
  // (global_load_lds_dwordx4: lane l of a copy writes the 16 bytes at LDS
  // offset 16 l of a 1 KB block, i.e. sixteen 64-byte slab rows), so no
  // staging registers and no LDS store instructions are involved.  A stage
  // holds M/16 blocks of A rows then N/16 blocks of B rows; block b holds
  // rows 16b..16b+15, and lane l fills row 16b + l/4 at position l%4, which
  // holds logical chunk (l%4) ^ (row/4 % 4).  Wave w issues blocks w, w+4,
  // w+8, ..; each copy's scalar base (its column range's weight matrix: a
  // block never straddles two ranges, whose starts are multiples of 16) and
  // each lane's offset are fixed for the whole K loop (rows clamped into the
  // matrix: rows past M or N only feed outputs that are never stored), and
  // the slab's k offset moves the scalar base.
  const bf16 *qbase[NQ];
  uint32_t doff[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int blk = wave + 4 * q;
    if (q < ABLK / 4) {
      const int row = 16 * blk + (lane >> 2);
      const int j = (lane & 3) ^ ((row >> 2) & 3);
      qbase[q] = A + (int64_t)m0 * p.lda;
      doff[q] = (uint32_t)(((int64_t)min(row, p.M - 1 - m0) * p.lda + j * 8) * (int64_t)sizeof(bf16));
    } else {
      const int rt = 16 * (blk - ABLK);                     // block's first row within the tile
      const int row = rt + (lane >> 2);
      const int j = (lane & 3) ^ ((row >> 2) & 3);
      const int s = seg_of(p, min(n0 + rt, p.N - 1));       // uniform: one range per block
      const int nb = SEG_FIELD(p, s, n_begin);
      const int64_t ldb = SEG_FIELD(p, s, ldb);
      qbase[q] = reinterpret_cast<const bf16 *>(SEG_FIELD(p, s, B));
      doff[q] = (uint32_t)(((int64_t)(min(n0 + row, p.N - 1) - nb) * ldb + j * 8) * (int64_t)sizeof(bf16));
    }
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16 *)lds;
  // Scalar operands of the copies of one slab (global base per copy, LDS
  // block address for M0), formed before the MFMAs they are spread over, so
  // that a copy between two MFMAs is just an M0 write and the copy itself.
  struct SlabOps {
    const bf16 *src[NQ];
    uint32_t dst[NQ];
  };
  auto slab_ops = [&](int kt, SlabOps &o) {
    const uint32_t stage = lds_base + (kt % GB_NST) * (BT::STAGE * 2);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      o.src[q] = uniform_ptr(qbase[q] + kt * GB_K);
      o.dst[q] = __builtin_amdgcn_readfirstlane(stage + (wave + 4 * q) * 1024);
    }
  };
#define GB_COPY(O, Q)                                                           \
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"            \
               :: "v"(doff[Q]), "s"((O).src[Q]), "s"((O).dst[Q]) : "memory", "m0")

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto load_frags = [&](int kt, int kk, bf16x8 *a, bf16x8 *b) {
    const bf16 *As = lds + (kt % GB_NST) * BT::STAGE, *Bs = As + BT::M * GB_K;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      a[i] = *reinterpret_cast<const bf16x8 *>(&As[swz(wm * 32 * TM + i * 32 + l32, kk + g * 8)]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      b[j] = *reinterpret_cast<const bf16x8 *>(&Bs[swz(wn * 32 * TN + j * 32 + l32, kk + g * 8)]);
  };
  // the TM x TN MFMAs of one k-step; with DMA_KT >= 0, copies of that slab go
  // between rows of MFMAs: the first k-step of an interval (H = 0) issues
  // copies 0..QH-1, the second QH..NQ-1 (a copy instruction stalls its wave
  // until the address unit takes it; between MFMAs the stall overlaps the
  // matrix pipe instead of idling it)
  auto mma = [&](const bf16x8 *a, const bf16x8 *b, const SlabOps *ops, int h) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      if (ops) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int lo = h * QH + (i * QH) / TM, hi = h * QH + ((i + 1) * QH) / TM;
          if (q >= lo && q < hi && q < (h + 1) * QH) GB_COPY(*ops, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Pipeline over barrier intervals j: the interval runs k-step 16..31 of
  // slab j and k-step 0..15 of slab j+1 (whose fragments are read from LDS
  // while the previous MFMAs run), copies slab j+NST into the stage slab j
  // used (free once every wave passed barrier j: a wave's LDS reads are
  // complete at its barrier), then waits for slab j+2.  The main loop always
  // copies (constant wait, no branches); the last intervals only drain.
  SlabOps ops;
#pragma unroll
  for (int c = 0; c < GB_NST; ++c)
    if (c < nk) {
      slab_ops(c, ops);
#pragma unroll
      for (int q = 0; q < NQ; ++q) GB_COPY(ops, q);
    }
  bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
  // slab 0 landed: at most slabs 1..NST-1 outstanding
  wait_slabs_outstanding<NQ>(min(nk, GB_NST) - 1);
  __syncthreads();
  load_frags(0, 0, a0, b0);
  load_frags(0, 16, a1, b1);
  __builtin_amdgcn_sched_barrier(0);
  mma(a0, b0, nullptr, 0);
  __builtin_amdgcn_sched_barrier(0);
  // slab 1 landed
  wait_slabs_outstanding<NQ>(min(nk, GB_NST) - 2);
  __syncthreads();
  int j = 0;
  for (; j + GB_NST < nk; ++j) {
    slab_ops(j + GB_NST, ops);
    load_frags(j + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1, &ops, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(j + 1, 16, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0, &ops, 1);
    __builtin_amdgcn_sched_barrier(0);
    // slab j+2 landed: slabs j+3 .. j+NST may stay outstanding
    __builtin_amdgcn_s_waitcnt(GB_VMCNT((GB_NST - 2) * NQ));
    __syncthreads();
  }
  for (; j + 1 < nk; ++j) {
    load_frags(j + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1, nullptr, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_frags(j + 1, 16, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0, nullptr, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_slabs_outstanding<NQ>(nk - 1 - (j + 2));
    __syncthreads();
  }
  mma(a1, b1, nullptr, 0);  // k-step 16..31 of the last slab
#undef GB_COPY

  // epilogue through LDS (the operand stages are free after the last barrier)
  bf16 *Cs = lds;
  // Channel-major ranges are aligned to the tile on the host, so a tile is
  // either all row-major or all channel-major.
  const int st0 = seg_of(p, min(n0, p.N - 1));
  if (!SEG_FIELD(p, st0, tr)) {
    // consumer of a split RMSNorm: row m of the product is scaled by
    // 1 / sqrt(mean of the squares of its normalised input row + eps), the
    // producer's 64-column partial sums added in column order
    __shared__ float rs_s[BT::M];
    if (p.rs_part) {
      for (int row = tid; row < BT::M; row += GB_THREADS) {
        const float *pp = p.rs_part + (int64_t)min(m0 + row, p.M - 1) * p.rs_chunks;
        float ss = 0.f;
        if ((p.rs_chunks & 3) == 0) {  // 16-byte loads, the same order
          for (int j = 0; j < p.rs_chunks; j += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(pp + j);
            ss += v.x;
            ss += v.y;
            ss += v.z;
            ss += v.w;
          }
        } else {
          for (int j = 0; j < p.rs_chunks; ++j) ss += pp[j];
        }
        rs_s[row] = 1.0f / sqrtf(ss / (float)(64 * p.rs_chunks) + p.rs_eps);
      }
      __syncthreads();
    }
    // A lane's rows of row block i are 8q + 4g + e (q, e < 4): their scale
    // factors are read as four 16-byte words ahead of the block's LDS stores,
    // so no store waits on a read.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float rsv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v = make_float4(1.f, 1.f, 1.f, 1.f);
        if (p.rs_part) v = *reinterpret_cast<const float4 *>(&rs_s[wm * 32 * TM + i * 32 + 8 * q + 4 * g]);
        rsv[4 * q] = v.x;
        rsv[4 * q + 1] = v.y;
        rsv[4 * q + 2] = v.z;
        rsv[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 * TM + i * 32 + acc_row(r, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          Cs[row * BT::CPITCH + wn * 32 * TN + j * 32 + l32] = (bf16)(acc[i][j][r] * rsv[r]);
      }
    }
    __syncthreads();
    // producer of a split RMSNorm: per row, the sum of squares of the stored
    // values of each 64-column chunk of [0, rn_cols) in this tile
    if (p.rn_part && n0 < p.rn_cols) {
      const int nch = min(BT::N, p.rn_cols - n0) / 64, chunks = p.rn_cols / 64;
      for (int row = tid; row < BT::M; row += GB_THREADS) {
        if (m0 + row >= p.M) continue;
        for (int j = 0; j < nch; ++j) {
          float ss = 0.f;
#pragma unroll
          for (int c8 = 0; c8 < 64; c8 += 8) {
            const bf16x8 v = *reinterpret_cast<const bf16x8 *>(&Cs[row * BT::CPITCH + j * 64 + c8]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf((float)v[e], (float)v[e], ss);
          }
          p.rn_part[(int64_t)(m0 + row) * chunks + n0 / 64 + j] = ss;
        }
      }
    }
    // Stores: 8-column runs, U passes at a time (their LDS reads issued
    // together).  Row m goes to row (b H + h) S + s of its range's output
    // (b = m / S, s = m % S, h the head of the column).
    constexpr int RUNS = BT::N / 8, PASSES = BT::M * RUNS / GB_THREADS;
    static_assert(BT::M * RUNS % GB_THREADS == 0, "runs must split evenly over the threads");
    constexpr int U = PASSES % 8 == 0 ? 8 : PASSES % 6 == 0 ? 6 : PASSES % 4 == 0 ? 4 : 1;
    if (st0 == p.rope_seg) {
      // A rotated range (its tiles hold whole heads, dh a multiple of 16, at
      // most 128): a unit is 8 pairs of one row -- columns c..c+7 with their
      // partners c+dh/2.. (half-split) or the 16 columns c..c+15
      // (interleaved) -- in every head of the tile, rotated by the row's
      // cos / sin of those pairs from the table and stored as 8-column runs.
      // A thread's units (at most 8) have their table values loaded first.
      const int dh = SEG_FIELD(p, st0, dh), P = dh >> 1, upr = dh >> 4;  // units per head row
      const int64_t ld = SEG_FIELD(p, st0, ld);
      bf16 *cb = reinterpret_cast<bf16 *>(SEG_FIELD(p, st0, C)) + SEG_FIELD(p, st0, off);
      const int h0 = (n0 - SEG_FIELD(p, st0, n_begin)) / dh;  // the tile's first head
      const int nh = min(BT::N, p.N - n0) / dh;                // heads in the tile
      const int nunit = BT::M * upr;
      // (formed here: hoisted to the kernel's start, values derived from the
      // thread index would occupy a register through the K loop)
      int tid_r = tid;
      asm volatile("" : "+v"(tid_r));
      constexpr int MAXU = BT::M * 8 / GB_THREADS;
      float4 tcs[MAXU][4];
#pragma unroll
      for (int it = 0; it < MAXU; ++it) {
        const int u = tid_r + GB_THREADS * it;
        if (u < nunit) {
          const int row = u / upr, k = u - row * upr;
          const float *tb = p.rope_tab + (int64_t)min(m0 + row, p.M - 1) * dh + 8 * k;
          tcs[it][0] = *reinterpret_cast<const float4 *>(tb);
          tcs[it][1] = *reinterpret_cast<const float4 *>(tb + 4);
          tcs[it][2] = *reinterpret_cast<const float4 *>(tb + P);
          tcs[it][3] = *reinterpret_cast<const float4 *>(tb + P + 4);
        }
      }
#pragma unroll
      for (int it = 0; it < MAXU; ++it) {
        const int u = tid_r + GB_THREADS * it;
        if (u >= nunit) break;
        const int row = u / upr, k = u - row * upr;
        const int m = m0 + row;
        if (m >= p.M) continue;
        const float co[8] = {tcs[it][0].x, tcs[it][0].y, tcs[it][0].z, tcs[it][0].w,
                             tcs[it][1].x, tcs[it][1].y, tcs[it][1].z, tcs[it][1].w};
        const float si[8] = {tcs[it][2].x, tcs[it][2].y, tcs[it][2].z, tcs[it][2].w,
                             tcs[it][3].x, tcs[it][3].y, tcs[it][3].z, tcs[it][3].w};
        const int ca = p.rope_conv ? 16 * k : 8 * k, cbb = ca + (p.rope_conv ? 8 : P);  // within a head
        const int b = m / p.S, sq = m - b * p.S;
        bf16 *dst = cb + ((int64_t)(b * p.H + h0) * p.S + sq) * ld;
        const int64_t hstep = (int64_t)p.S * ld;  // next head, same token
        for (int hh = 0; hh < nh; ++hh, dst += hstep) {
          bf16x8 va = *reinterpret_cast<const bf16x8 *>(&Cs[row * BT::CPITCH + hh * dh + ca]);
          bf16x8 vb = *reinterpret_cast<const bf16x8 *>(&Cs[row * BT::CPITCH + hh * dh + cbb]);
          float ra, rb;
          if (p.rope_conv == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              rope_rot((float)va[j], (float)vb[j], co[j], si[j], ra, rb);
              va[j] = (bf16)ra;
              vb[j] = (bf16)rb;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              rope_rot((float)va[2 * j], (float)va[2 * j + 1], co[j], si[j], ra, rb);
              va[2 * j] = (bf16)ra;
              va[2 * j + 1] = (bf16)rb;
              rope_rot((float)vb[2 * j], (float)vb[2 * j + 1], co[4 + j], si[4 + j], ra, rb);
              vb[2 * j] = (bf16)ra;
              vb[2 * j + 1] = (bf16)rb;
            }
          }
          *reinterpret_cast<bf16x8 *>(dst + ca) = va;
          *reinterpret_cast<bf16x8 *>(dst + cbb) = vb;
        }
      }
    } else if constexpr (GB_THREADS % RUNS == 0) {
      // a thread keeps one run of columns; its rows step by RSTEP
      constexpr int RSTEP = GB_THREADS / RUNS;
      const int cc = tid % RUNS, r0 = tid / RUNS;
      const int n = n0 + cc * 8;
      if (n < p.N) {
        const int s = seg_of(p, n);
        const int nn = n - SEG_FIELD(p, s, n_begin), dh = SEG_FIELD(p, s, dh);
        const int h = nn / dh, d = nn - h * dh;
        const int64_t ld = SEG_FIELD(p, s, ld);
        bf16 *cb = reinterpret_cast<bf16 *>(SEG_FIELD(p, s, C)) + SEG_FIELD(p, s, off) + d;
        const int m = m0 + r0, b = m / p.S, sq = m - b * p.S;
        bf16 *dst = cb + ((int64_t)(b * p.H + h) * p.S + sq) * ld;
        const int64_t wrap = (int64_t)(p.H - 1) * p.S * ld;
        if (p.rn_gain && n < p.rn_cols) {  // the producer stores its normalised columns times the gains
          const bf16x8 gv = *reinterpret_cast<const bf16x8 *>(p.rn_gain + n);
          store_row_runs<PASSES, U, RSTEP, BT::CPITCH, true>(Cs, r0, cc, dst, ld, m, p.M, sq, p.S, wrap, gv);
        } else {
          store_row_runs<PASSES, U, RSTEP, BT::CPITCH, false>(Cs, r0, cc, dst, ld, m, p.M, sq, p.S, wrap, bf16x8{});
        }
      }
    } else {
      for (int it = 0; it < PASSES; it += U) {
        bf16x8 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = tid + GB_THREADS * (it + u);
          const int row = c / RUNS, cc = c - row * RUNS;
          v[u] = *reinterpret_cast<const bf16x8 *>(&Cs[row * BT::CPITCH + cc * 8]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = tid + GB_THREADS * (it + u);
          const int row = c / RUNS, cc = c - row * RUNS;
          const int m = m0 + row, n = n0 + cc * 8;
          if (m >= p.M || n >= p.N) continue;
          const int s = seg_of(p, n);
          const int nn = n - SEG_FIELD(p, s, n_begin), dh = SEG_FIELD(p, s, dh);
          const int h = nn / dh, d = nn - h * dh;
          const int b = m / p.S, sq = m - b * p.S;
          bf16 *dst = reinterpret_cast<bf16 *>(SEG_FIELD(p, s, C)) +
                      ((int64_t)(b * p.H + h) * p.S + sq) * SEG_FIELD(p, s, ld) + SEG_FIELD(p, s, off) + d;
          if (p.rn_gain && n < p.rn_cols) {  // the producer stores its normalised columns times the gains
            const bf16x8 gv = *reinterpret_cast<const bf16x8 *>(p.rn_gain + n);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[u][e] = (bf16)((float)v[u][e] * (float)gv[e]);
          }
          *reinterpret_cast<bf16x8 *>(dst) = v[u];
        }
      }
    }
  } else {
    // Channel-major destination: the tile goes to LDS transposed (column n
    // holds the tile's rows, i.e. tokens, contiguously).  A lane's
    // accumulators hold four consecutive rows of one column, written as one
    // 8-byte store; then lanes take consecutive 8-token runs of one column,
    // so a half wave writes 512 consecutive bytes of the output.
    constexpr int TP = BT::M + 8;  // transposed pitch (elements)
    static_assert(BT::N * TP <= BT::LDS, "transposed tile must fit the LDS area");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // acc rows 8q + 4g .. +3 (acc_row of r = 4q .. 4q+3) of column l32
          bf16 v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)acc[i][j][4 * q + e];
          *reinterpret_cast<uint2 *>(&Cs[(wn * 32 * TN + j * 32 + l32) * TP + wm * 32 * TM + i * 32 +
                                         acc_row(4 * q, lane)]) = *reinterpret_cast<const uint2 *>(v4);
        }
    __syncthreads();
    // Column n's run of tokens m .. m+7 goes to row (b H + h) dh + d = b H dh
    // + (n - range start) of its range, at token s (b = m / S, s = m % S).
    bf16 *t_C = reinterpret_cast<bf16 *>(SEG_FIELD(p, st0, C));
    const int t_dh = SEG_FIELD(p, st0, dh), t_nb = SEG_FIELD(p, st0, n_begin);
    constexpr int RG = BT::M / 8, TPASSES = BT::M * BT::N / 8 / GB_THREADS;  // 8-token runs per column
    static_assert(BT::M * BT::N / 8 % GB_THREADS == 0, "runs must split evenly over the threads");
    constexpr int TU = TPASSES % 8 == 0 ? 8 : TPASSES % 4 == 0 ? 4 : 1;
    bool tfast = false;
    if constexpr (GB_THREADS % RG == 0) {
      // a thread keeps one run of tokens; its columns step by CSTEP, U passes
      // at a time (their LDS reads issued together)
      constexpr int CSTEP = GB_THREADS / RG;
      const int rg = tid % RG, col0 = tid / RG;
      const int m = m0 + rg * 8;
      const int b = m / p.S, sq = m - b * p.S;
      tfast = m + 8 <= p.M && sq + 8 <= p.S;
      if (tfast) {
        bf16 *dst = t_C + ((int64_t)b * p.H * t_dh + (n0 + col0 - t_nb)) * p.S + sq;
        for (int it = 0; it < TPASSES; it += TU) {
          uint4 v[TU];
#pragma unroll
          for (int u = 0; u < TU; ++u)
            v[u] = *reinterpret_cast<const uint4 *>(&Cs[(col0 + CSTEP * (it + u)) * TP + rg * 8]);
#pragma unroll
          for (int u = 0; u < TU; ++u)
            if (n0 + col0 + CSTEP * (it + u) < p.N)
              *reinterpret_cast<uint4 *>(dst + (int64_t)(CSTEP * (it + u)) * p.S) = v[u];
        }
      }
    }
    if (!tfast) {
      for (int it = 0; it < TPASSES; ++it) {
        const int c = tid + GB_THREADS * it;
        const int col = c / RG, rg = c - col * RG;
        const int m = m0 + rg * 8, n = n0 + col;
        if (m >= p.M || n >= p.N) continue;
        const int b = m / p.S, sq = m - b * p.S;
        const bf16 *src = &Cs[col * TP + rg * 8];
        if (sq + 8 <= p.S && m + 8 <= p.M) {
          *reinterpret_cast<uint4 *>(t_C + ((int64_t)b * p.H * t_dh + (n - t_nb)) * p.S + sq) =
              *reinterpret_cast<const uint4 *>(src);
        } else {
          for (int e = 0; e < 8 && m + e < p.M; ++e) {
            const int me = m + e, be = me / p.S, se = me - be * p.S;
            t_C[((int64_t)be * p.H * t_dh + (n - t_nb)) * p.S + se] = src[e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Skinny bf16 kernel for decode (M <= 64 rows, weights streamed once).
//
// With one token per sequence the projections are weight-bandwidth bound:
// every weight element is used by at most 64 rows.  A 256-thread workgroup
// owns a 64x128 output tile and one K slice; the grid covers the N tiles times
// a split of K chosen on the host.  Slices write fp32 partial tiles; a second
// kernel adds the slices in a fixed order (deterministic) and applies the
// column-range store mapping.  Operand chunks of 128 k values (256 bytes of
// every row) are copied global -> LDS with global_load_lds through SK_NST
// stages: one copy instruction moves four whole 256-byte row pieces, so each
// weight row is fetched in long contiguous runs rather than scattered
// 128-byte pieces, which keeps HBM pages open across the request.
#ifndef SK_STAGES
#define SK_STAGES 3
#endif
constexpr int SK_M = 64, SK_N = 128, SK_K = 128, SK_NST = SK_STAGES;
constexpr int SK_MMAX = 512;  // larger M goes to the large-tile kernel
constexpr int SK_STAGE = (SK_M + SK_N) * SK_K;    // elements per stage
constexpr int SK_CPW = (SK_M + SK_N) / 4 / 4;      // copy instructions per wave per chunk
// LDS position of element (r, k) of a stage operand: 128-element rows whose
// 16-byte pieces are XOR-permuted by the row index, so the 32 consecutive rows
// one MFMA fragment read touches fall in distinct banks.
__device__ inline int swz_sk(int r, int k) {
  return r * SK_K + ((((k >> 3) ^ r) & 15) << 3) + (k & 7);
}

// Output column n (in column range st) of batch z under the column-range
// mapping (head-major rows, optionally transposed); element (m, n) goes to
// C + at(m).
struct SkinnyCol {
  bf16 *C;
  int64_t ld, h, d, dh;
  bool tr;
  __device__ SkinnyCol(const GemmParams &p, int z, int st, int n) {
    const int nn = n - SEG_FIELD(p, st, n_begin);
    dh = SEG_FIELD(p, st, dh);
    h = nn / dh;
    d = nn - h * dh;
    tr = SEG_FIELD(p, st, tr);
    ld = SEG_FIELD(p, st, ld);
    C = reinterpret_cast<bf16 *>(SEG_FIELD(p, st, C)) + (int64_t)z * p.strideC +
        (tr ? 0 : SEG_FIELD(p, st, off) + d);
  }
  __device__ void store(const GemmParams &p, int m, float v) const {
    const int b = m / p.S, sq = m - b * p.S;
    const int64_t at = tr ? ((b * p.H + h) * dh + d) * p.S + sq : ((b * p.H + h) * p.S + sq) * ld;
    C[at] = (bf16)v;
  }
};

__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p, float *part, int kslice) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[SK_NST * SK_STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds M0
  const int g = lane >> 5, l32 = lane & 31;
  // grid z: batch index times the 64-row blocks of M
  const int mblocks = (p.M + SK_M - 1) / SK_M;
  const int z = blockIdx.z / mblocks, m0 = (blockIdx.z - z * mblocks) * SK_M;
  const int n0 = blockIdx.x * SK_N, ks = blockIdx.y;
  const int k_begin = ks * kslice;
  const int nk = kslice / SK_K;
  const bf16 *A = reinterpret_cast<const bf16 *>(p.A) + (int64_t)z * p.strideA + (int64_t)m0 * p.lda +
                  k_begin;
  // B rows: column ranges start at multiples of 128 (checked on the host)
  const int st = seg_of(p, n0);
  const int t_nb = SEG_FIELD(p, st, n_begin);
  const int64_t t_ldb = SEG_FIELD(p, st, ldb);
  const bf16 *Bb = reinterpret_cast<const bf16 *>(SEG_FIELD(p, st, B)) + (int64_t)z * p.strideB +
                   (int64_t)(n0 - t_nb) * t_ldb + k_begin;

  // Copy blocks of a chunk: 16 of A (rows 4b..4b+3) then 32 of B; wave w
  // issues blocks w, w+4, ..  Lane l fills row 4b + l/16 at position l%16,
  // which holds logical 16-byte piece (l%16) ^ (row % 16).  Rows past M or N
  // are clamped (they only feed outputs that are never stored).
  uint32_t doff[SK_CPW];
#pragma unroll
  for (int q = 0; q < SK_CPW; ++q) {
    const int blk = wave + 4 * q;  // 0..47
    const bool is_a = blk < SK_M / 4;
    const int row = 4 * (is_a ? blk : blk - SK_M / 4) + (lane >> 4);
    const int j = (lane & 15) ^ (row & 15);
    const int rc = is_a ? min(row, p.M - 1 - m0) : min(row, p.N - 1 - n0);
    const int64_t ld = is_a ? p.lda : t_ldb;
    doff[q] = (uint32_t)((rc * ld + j * 8) * (int64_t)sizeof(bf16));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16 *)lds;
#define SK_DMA(KK, STG)                                                               \
  do {                                                                                \
    const bf16 *a_ = uniform_ptr(A + (KK)), *b_ = uniform_ptr(Bb + (KK));             \
    _Pragma("unroll") for (int q = 0; q < SK_CPW; ++q) {                              \
      const int blk = wave + 4 * q;                                                   \
      const uint32_t m0_ =                                                            \
          __builtin_amdgcn_readfirstlane(lds_base + (STG) * (SK_STAGE * 2) + blk * 1024); \
      if (blk < SK_M / 4)                                                             \
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"             \
                     :: "v"(doff[q]), "s"(a_), "s"(m0_) : "memory", "m0");            \
      else                                                                            \
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"             \
                     :: "v"(doff[q]), "s"(b_), "s"(m0_) : "memory", "m0");            \
    }                                                                                 \
  } while (0)

  // wave tile: rows (wave / 2) * 32, columns (wave % 2) * 64 (two 32x32 tiles)
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc0, acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;

#pragma unroll
  for (int c = 0; c < SK_NST - 1; ++c)
    if (c < nk) SK_DMA(c * SK_K, c);
  int cs = 0;  // stage of chunk kt
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's copies of chunk kt have landed once at most the later
    // chunks already issued (up to SK_NST - 2 of them) are outstanding; the
    // barrier publishes every wave's copies and frees the stage read in the
    // previous iteration for chunk kt + SK_NST - 1
    const int later = min(nk - 1 - kt, SK_NST - 2);
    if (later >= SK_NST - 2) __builtin_amdgcn_s_waitcnt(GB_VMCNT(SK_CPW * (SK_NST - 2)));
    else if (SK_NST > 3 && later == 2) __builtin_amdgcn_s_waitcnt(GB_VMCNT(2 * SK_CPW));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(GB_VMCNT(SK_CPW));
    else __builtin_amdgcn_s_waitcnt(GB_VMCNT(0));
    __syncthreads();
    if (kt + SK_NST - 1 < nk) SK_DMA((kt + SK_NST - 1) * SK_K, cs == 0 ? SK_NST - 1 : cs - 1);
    const bf16 *As = lds + cs * SK_STAGE, *Bs = As + SK_M * SK_K;
    cs = cs == SK_NST - 1 ? 0 : cs + 1;
#pragma unroll
    for (int kk = 0; kk < SK_K; kk += 16) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&As[swz_sk(wm * 32 + l32, kk + g * 8)]);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(&Bs[swz_sk(wn * 64 + l32, kk + g * 8)]);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(&Bs[swz_sk(wn * 64 + 32 + l32, kk + g * 8)]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
    }
  }
#undef SK_DMA
  // without a split of K the tile is final: store bf16 through the mapping;
  // otherwise an fp32 partial tile [z][ks][M][N] for the reduce kernel
  const int n = n0 + wn * 64 + l32;
  if (gridDim.y == 1) {
    // the 128 columns of a tile lie in one column range (st)
    const SkinnyCol c0(p, z, st, min(n, p.N - 1)), c1(p, z, st, min(n + 32, p.N - 1));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 32 + acc_row(r, lane);
      if (m < p.M) {
        if (n < p.N) c0.store(p, m, acc0[r]);
        if (n + 32 < p.N) c1.store(p, m, acc1[r]);
      }
    }
    return;
  }
  float *pt = part + (((int64_t)z * gridDim.y + ks) * p.M) * p.N;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm * 32 + acc_row(r, lane);
    if (m < p.M) {
      if (n < p.N) pt[(int64_t)m * p.N + n] = acc0[r];
      if (n + 32 < p.N) pt[(int64_t)m * p.N + n + 32] = acc1[r];
    }
  }
}

// Sum the K slices in order and store through the column-range mapping.
__global__ __launch_bounds__(256) void gemm_skinny_reduce(GemmParams p, const float *part,
                                                          int nsplit) {
  const int z = blockIdx.y;
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int m = (int)(i / p.N), n = (int)(i - (int64_t)m * p.N);
    const float *src = part + (int64_t)z * nsplit * total + i;
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) acc += src[(int64_t)s * total];
    SkinnyCol(p, z, seg_of(p, n), n).store(p, m, acc);
  }
}

}  // namespace

// Split of K the skinny kernel uses for an M <= 64 product: the largest
// divisor of K/128 that keeps the grid within one workgroup per CU (a stage
// set fills most of a CU's LDS, and a second round of workgroups would leave
// the tail of the launch running on a fraction of the chip).
static int skinny_split(int M, int N, int K, int batch) {
  const int ntile = (N + SK_N - 1) / SK_N, mblocks = (M + SK_M - 1) / SK_M;
  const int kchunks = K / SK_K;
  const int want = std::max(1, 256 / (ntile * batch * mblocks));
  int nsplit = 1;
  for (int c = 1; c <= kchunks; ++c)
    if (kchunks % c == 0 && c <= want) nsplit = c;
  return nsplit;
}

size_t gemm_scratch_bytes(int dtype, int M, int N, int K, int batch) {
  if (dtype != BF16 || M > SK_MMAX || K % SK_K != 0) return 0;
  const int nsplit = skinny_split(M, N, K, batch);
  return nsplit > 1 ? (size_t)nsplit * batch * M * N * sizeof(float) : 0;
}

// Compute units of the current device (one resident large-tile workgroup each).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// A big-kernel tile must not mix row-major and channel-major column ranges.
static bool tr_aligned(const GemmDesc &d, int bn) {
  for (int i = 1; i < d.nseg; ++i)
    if (d.seg[i].tr != d.seg[i - 1].tr && d.seg[i].n_begin % bn != 0) return false;
  return true;
}

template <int TM, int TN, int NST = GB_STAGES>
static hipError_t launch_big(const GemmParams &p, const GemmDesc &d, int n_lo, int n_hi, hipStream_t st) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  const int tm = (d.M + BM - 1) / BM, tn = (n_hi - n_lo + BN - 1) / BN;
  const int T = tm * tn;
  // Tiles of an XCD walk groups of group_m tile rows: at four, the 32 tiles
  // an XCD runs at once cover 4 row and 8 column panels (the fewest for 32),
  // measured best for K >= 1536 (eight: +1% on the out- and down-
  // projections, sixteen: +37%); short K runs one tile row at a time.
  const int group_m = d.K <= 1024 ? 1 : 4;
  // With a rotated column range (whose tiles take longer) the tile columns
  // are visited with a stride coprime to their count, so that every XCD's
  // contiguous share of tiles holds its part of that range instead of some
  // XCDs getting all of it (same panels per group, so the same L2 reuse).
  int cstride = 1;
  if (p.rope_tab)
    for (int s : {5, 7, 11, 13})
      if (s < tn && std::gcd(s, tn) == 1) {
        cstride = s;
        break;
      }
  hipLaunchKernelGGL((gemm_big_kernel<TM, TN, NST>), dim3(T), dim3(GB_THREADS), 0, st, p, tm, tn, n_lo,
                     (T % 8 == 0) ? 1 : 0, group_m, cstride);
  return hipGetLastError();
}

bool gemm_uses_large_tiles(const GemmDesc &d) {
  bool big = d.dtype == BF16 && !d.b_kn && !d.a_km && d.batch == 1 && d.K % GB_K == 0 && d.M >= 512 &&
             d.N % 8 == 0 && (int64_t)d.M * d.lda < (1LL << 31);
  for (int i = 0; i < d.nseg && big; ++i)
    big = d.seg[i].n_begin % 16 == 0 && (int64_t)d.N * d.seg[i].ldb < (1LL << 31);
  return big && tr_aligned(d, BigTile<4, 4, GB_STAGES>::N);
}

// The large-tile configuration launch_gemm runs a product on: 0 for 256x256
// tiles, 1 for 192x192, 2 for 256x128.
//  * A product whose 256x256 tiles would leave most CUs idle in its only
//    round (the down projection: 144 tiles) runs as 192x192 tiles, which
//    fill one round (242 tiles) at a somewhat lower efficiency per tile.
//  * Short K (the kv up-projection, K = 512): 256x128 tiles through three
//    stages fit two workgroups per CU (two waves per SIMD), so one's
//    epilogue runs under the other's K loop (5% faster there; slower for
//    long K, whose tiles are all main loop).
static int big_config(const GemmDesc &d) {
  const int cus = device_cus();
  const int64_t t256 = (int64_t)((d.M + 255) / 256) * ((d.N + 255) / 256);
  const int64_t t192 = (int64_t)((d.M + 191) / 192) * ((d.N + 191) / 192);
  if (10 * t256 <= 6 * cus && t192 <= cus && tr_aligned(d, 192)) return 1;
  if (d.K <= 512 && tr_aligned(d, 128)) return 2;
  return 0;
}

bool gemm_rope_fusable(const GemmDesc &d, int seg) {
  if (seg < 0 || seg >= d.nseg || !gemm_uses_large_tiles(d)) return false;
  static const int tile_n[3] = {256, 192, 128};
  const int bn = tile_n[big_config(d)];
  const GemmSeg &s = d.seg[seg];
  const int end = seg + 1 < d.nseg ? d.seg[seg + 1].n_begin : d.N;
  return !s.tr && s.dh % 16 == 0 && s.dh <= 128 && bn % s.dh == 0 && s.n_begin % bn == 0 &&
         (end - s.n_begin) % s.dh == 0 && (end == d.N || end % bn == 0) &&
         !(d.rn_part && s.n_begin < d.rn_cols);
}

bool gemm_takes_large_tiles(int dtype, int M, int N, int K) {
  return dtype == BF16 && K % GB_K == 0 && M >= 512 && N % 8 == 0 && (int64_t)M * K < (1LL << 31) &&
         (int64_t)N * K < (1LL << 31);
}

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
  p.rn_part = d.rn_part;
  p.rn_gain = reinterpret_cast<const bf16 *>(d.rn_gain);
  p.rn_cols = d.rn_cols;
  p.rs_part = d.rs_part;
  p.rs_chunks = d.rs_chunks;
  p.rs_eps = d.rs_eps;
  p.rope_tab = d.rope_tab;
  p.rope_seg = d.rope_tab ? d.rope_seg : -1;
  p.rope_conv = d.rope_conv;
  if (d.rope_tab && !gemm_rope_fusable(d, d.rope_seg)) return hipErrorInvalidValue;
  if (gemm_uses_large_tiles(d)) {
    const int cfg = big_config(d);
    if (cfg == 1) return launch_big<3, 3>(p, d, 0, d.N, st);
    if (cfg == 2) return launch_big<4, 2, 3>(p, d, 0, d.N, st);
    return launch_big<4, 4>(p, d, 0, d.N, st);
  }
  // a split RMSNorm exists only in the large-tile kernel's epilogue
  if (d.rn_part || d.rs_part) return hipErrorInvalidValue;
  bool skinny = d.dtype == BF16 && !d.b_kn && !d.a_km && d.M <= SK_MMAX && d.K % SK_K == 0 && d.N % 8 == 0 &&
                d.batch * ((d.M + SK_M - 1) / SK_M) <= 65535;
  for (int i = 0; i < d.nseg && skinny; ++i) skinny = d.seg[i].n_begin % SK_N == 0;
  if (skinny) {
    // K is split only into a workspace big enough for the fp32 partials
    const int ntile = (d.N + SK_N - 1) / SK_N, mblocks = (d.M + SK_M - 1) / SK_M;
    int nsplit = skinny_split(d.M, d.N, d.K, d.batch);
    if (nsplit > 1 && (d.workspace == nullptr ||
                       (size_t)nsplit * d.batch * d.M * d.N * sizeof(float) > d.workspace_bytes))
      nsplit = 1;
    {
      float *part = reinterpret_cast<float *>(d.workspace);
      hipLaunchKernelGGL(gemm_skinny_kernel, dim3(ntile, nsplit, d.batch * mblocks), dim3(256), 0, st,
                         p, part, d.K / nsplit);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || nsplit == 1) return e;
      const int64_t total = (int64_t)d.M * d.N;
      const unsigned rb = (unsigned)std::min<int64_t>((total + 255) / 256, 2048);
      hipLaunchKernelGGL(gemm_skinny_reduce, dim3(rb, d.batch), dim3(256), 0, st, p, part, nsplit);
      return hipGetLastError();
    }
  }
  dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM, d.batch);
  dim3 block(256);
#define MLA_GEMM_GENERIC(T_)                                                                  \
  if (d.a_km) {                                                                               \
    if (d.b_kn) hipLaunchKernelGGL((gemm_kernel<T_, true, true>), grid, block, 0, st, p);     \
    else hipLaunchKernelGGL((gemm_kernel<T_, false, true>), grid, block, 0, st, p);           \
  } else {                                                                                    \
    if (d.b_kn) hipLaunchKernelGGL((gemm_kernel<T_, true, false>), grid, block, 0, st, p);    \
    else hipLaunchKernelGGL((gemm_kernel<T_, false, false>), grid, block, 0, st, p);          \
  }
  if (d.dtype == BF16) {
    MLA_GEMM_GENERIC(bf16)
  } else {
    MLA_GEMM_GENERIC(float)
  }
#undef MLA_GEMM_GENERIC
  return hipGetLastError();
}

}  // namespace mla
