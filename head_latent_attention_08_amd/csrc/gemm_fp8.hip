// Block-scaled FP8 (OCP E4M3) projection products for gfx950.
//
// Following the FP8 scheme of the "Deep Seek V3" notes (section
// "infrastructure": fine-grained tile-wise / block-wise quantisation with
// online maxima, E4M3 everywhere, accumulation above FP8 precision):
//
// * Activations are quantised in 1 x 128 tiles along K, weights in 128 x 128
//   blocks.  Each tile's scale is a power of two 2^e, the smallest with
//   amax <= 448 * 2^e, stored as an E8M0 byte (e + 127).  The byte is the
//   block exponent the matrix cores take, so dequantisation costs nothing:
//   v_mfma_scale_f32_32x32x64_f8f6f4 multiplies each operand's 32-element
//   k-groups by 2^(byte - 127) and accumulates in fp32.
// * Scale bytes are stored k-block major: byte (kb, r) at s[kb * ld + r], one
//   per operand row (a weight block's exponent is repeated over its 128 rows),
//   so a tile's 256 row scales of one k-block are one 256-byte run.
//
// The product kernel keeps the structure of the bf16 large-tile kernel: a
// 256x256 output tile per 256-thread workgroup (four waves of 128x128), K in
// 64-byte slabs (64 fp8 values per row) copied global -> LDS by
// global_load_lds through four stages, two slabs of lead.  The 256 A-row and
// 256 B-row scale bytes of the slab's k-block ride with the slab as one more
// copy per wave (global_load_lds_dword: 64 lanes x 4 bytes), so every wave
// issues the same number of copies per slab and one vmcnt rule covers all.
// A slab is one MFMA k-step (32x32x64), so a slab carries twice the flops of
// a bf16 slab of the same bytes.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int F8_TILE = 128;                             // scale tile along K
constexpr int F8_BM = 256, F8_BN = 256, F8_BK = 64;      // output tile, k per slab (bytes)
constexpr int F8_NST = 4, F8_THREADS = 256;
constexpr int F8_NQ = (F8_BM + F8_BN) / 64;              // 1 KB operand copies per wave per slab
constexpr int F8_OPS = F8_NQ + 1;                        // plus one scale copy
constexpr int F8_OPB = (F8_BM + F8_BN) * F8_BK;          // operand bytes per stage
constexpr int F8_STAGE = F8_OPB + 1024;                  // + A scales, B scales, 512 spare
constexpr int F8_CPITCH = F8_BN + 8;                     // bf16 epilogue pitch (elements)
constexpr int F8_LDS = F8_NST * F8_STAGE > F8_BM * F8_CPITCH * 2 ? F8_NST * F8_STAGE : F8_BM * F8_CPITCH * 2;

// s_waitcnt immediate: at most n vector-memory operations outstanding
#define F8_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

template <int Q> __device__ inline void f8_wait_slabs(int slabs) {
  if (slabs >= 3) __builtin_amdgcn_s_waitcnt(F8_VMCNT(3 * Q));
  else if (slabs == 2) __builtin_amdgcn_s_waitcnt(F8_VMCNT(2 * Q));
  else if (slabs == 1) __builtin_amdgcn_s_waitcnt(F8_VMCNT(Q));
  else __builtin_amdgcn_s_waitcnt(F8_VMCNT(0));
}

// Byte offset of 16-byte chunk c of slab row r: 64-byte rows whose chunks are
// XOR-permuted by (r / 4) % 4 (16 consecutive rows read by a quarter wave
// fall in distinct banks).
__device__ inline int f8_swz(int r, int c) { return r * F8_BK + (((c ^ (r >> 2)) & 3) << 4); }

template <typename P> __device__ inline P *f8_uniform(P *q) {
  const uint64_t v = (uint64_t)q;
  return reinterpret_cast<P *>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                               (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}

struct Fp8GemmParams {
  const uint8_t *a, *sa, *b, *sb;
  int64_t lda, ld_sa, ldb, ld_sb, ldc;
  void *c;
  int M, N, K, c_f32;
  // column-range output mapping (bf16 C; c and ldc unused): nseg > 0
  int S = 1, H = 1, nseg = 0;
  GemmSeg seg[3];
};

__device__ inline int f8_seg_of(const Fp8GemmParams &p, int n) {
  return (p.nseg > 1 && n >= p.seg[1].n_begin) ? ((p.nseg > 2 && n >= p.seg[2].n_begin) ? 2 : 1) : 0;
}
// fields of column range s, read with constant indices only
#define F8_SEG(p, s, f) ((s) == 0 ? (p).seg[0].f : ((s) == 1 ? (p).seg[1].f : (p).seg[2].f))

__global__ __launch_bounds__(F8_THREADS) void fp8_gemm_kernel(Fp8GemmParams p, int tiles_m, int tiles_n,
                                                              int remap, int group_m) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[F8_LDS];

  // tile index: contiguous run per XCD, then grouped row-major order
  const int T = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (remap) t = (t & 7) * (T >> 3) + (t >> 3);
  const int per_group = group_m * tiles_n;
  const int grp = t / per_group;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int tm = first_m + (t % per_group) % gm;
  const int tn = (t % per_group) / gm;
  const int m0 = tm * F8_BM, n0 = tn * F8_BN;
  const int nk = p.K / F8_BK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  // Operand copies: block blk = wave + 4q holds 16 slab rows (A rows for
  // blk < 16, then B rows); lane l fills row 16 blk' + l/4 at chunk position
  // l % 4, which holds logical chunk (l % 4) ^ (row / 4 % 4).  Rows past M or
  // N are clamped into the matrix (they only feed outputs never stored).
  const uint8_t *qbase[F8_NQ];
  uint32_t doff[F8_NQ];
#pragma unroll
  for (int q = 0; q < F8_NQ; ++q) {
    const int blk = wave + 4 * q;
    const bool is_a = blk < F8_BM / 16;
    const int row = 16 * (is_a ? blk : blk - F8_BM / 16) + (lane >> 2);
    const int j = (lane & 3) ^ ((row >> 2) & 3);
    if (is_a) {
      qbase[q] = p.a + (int64_t)m0 * p.lda;
      doff[q] = (uint32_t)((int64_t)min(row, p.M - 1 - m0) * p.lda + j * 16);
    } else {
      qbase[q] = p.b + (int64_t)n0 * p.ldb;
      doff[q] = (uint32_t)((int64_t)min(row, p.N - 1 - n0) * p.ldb + j * 16);
    }
  }
  // Scale copy: waves 0 and 2 copy the A-row bytes of the tile, waves 1 and 3
  // the B-row bytes (256 bytes each; the copies of waves 2 and 3 land in the
  // spare area and are never read).
  const uint8_t *sbase = (wave & 1) ? p.sb + n0 : p.sa + m0;
  const int64_t sld = (wave & 1) ? p.ld_sb : p.ld_sa;
  const uint32_t soff = 4u * lane;

  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
  struct SlabOps {
    const uint8_t *src[F8_OPS];
    uint32_t dst[F8_OPS];
  };
  auto slab_ops = [&](int kt, SlabOps &o) __attribute__((always_inline)) {
    const uint32_t stage = lds_base + (kt % F8_NST) * F8_STAGE;
#pragma unroll
    for (int q = 0; q < F8_NQ; ++q) {
      o.src[q] = f8_uniform(qbase[q] + kt * F8_BK);
      o.dst[q] = __builtin_amdgcn_readfirstlane(stage + (wave + 4 * q) * 1024);
    }
    o.src[F8_NQ] = f8_uniform(sbase + (int64_t)(kt >> 1) * sld);
    o.dst[F8_NQ] = __builtin_amdgcn_readfirstlane(stage + F8_OPB + 256 * wave);
  };
#define F8_COPY(O, Q)                                                                        \
  do {                                                                                       \
    if ((Q) < F8_NQ)                                                                         \
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"                      \
                   :: "v"(doff[(Q) < F8_NQ ? (Q) : 0]), "s"((O).src[Q]), "s"((O).dst[Q])     \
                   : "memory", "m0");                                                        \
    else                                                                                     \
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"                        \
                   :: "v"(soff), "s"((O).src[Q]), "s"((O).dst[Q]) : "memory", "m0");         \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // A lane's fragment of a 32x32x64 step: row l32, the 32 k values of chunks
  // 2g and 2g + 1 (the same k mapping on both operands, so the pairing of k
  // values inside the instruction does not matter); its scale byte is the
  // row's exponent for the slab's k-block.
  struct Frags {
    i32x8 a[4], b[4];
    int sa[4], sb[4];
  };
  auto load_frags = [&](int kt, Frags &f) __attribute__((always_inline)) {
    const uint8_t *st = lds + (kt % F8_NST) * F8_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + l32;
      const uint4 lo = *reinterpret_cast<const uint4 *>(st + f8_swz(r, 2 * g));
      const uint4 hi = *reinterpret_cast<const uint4 *>(st + f8_swz(r, 2 * g + 1));
      f.a[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      f.sa[i] = st[F8_OPB + r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = F8_BM + wn * 128 + j * 32 + l32;
      const uint4 lo = *reinterpret_cast<const uint4 *>(st + f8_swz(r, 2 * g));
      const uint4 hi = *reinterpret_cast<const uint4 *>(st + f8_swz(r, 2 * g + 1));
      f.b[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      f.sb[j] = st[F8_OPB + 256 + wn * 128 + j * 32 + l32];
    }
  };
  // the 16 MFMAs of one slab; with ops, the slab's copies go between rows of
  // MFMAs (3, 2, 2, 2 per row)
  auto mma = [&](const Frags &f, const SlabOps *ops) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0,
                                                                    f.sa[i], 0, f.sb[j]);
      if (ops) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < F8_OPS; ++q) {
          const int lo = (i * F8_OPS + 3) / 4, hi = ((i + 1) * F8_OPS + 3) / 4;
          if (q >= lo && q < hi) F8_COPY(*ops, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Interval j: fragments of slab j+1 are read while slab j's MFMAs run and
  // slab j+NST is copied into the stage slab j used (every wave read slab j
  // before barrier j-1); then wait for slab j+2.
  SlabOps ops;
#pragma unroll
  for (int c = 0; c < F8_NST; ++c)
    if (c < nk) {
      slab_ops(c, ops);
#pragma unroll
      for (int q = 0; q < F8_OPS; ++q) F8_COPY(ops, q);
    }
  Frags f0, f1;
  f8_wait_slabs<F8_OPS>(min(nk, F8_NST) - 1);  // slab 0 landed
  __syncthreads();
  load_frags(0, f0);
  f8_wait_slabs<F8_OPS>(min(nk, F8_NST) - 2);  // slab 1 landed (and slab 0 read by all)
  __syncthreads();
  // one interval: MFMAs on cur while nxt receives slab jj+1; with copy, slab
  // jj+NST goes out (constant wait), else the pipeline drains
  auto interval = [&](int jj, Frags &cur, Frags &nxt, bool copy) __attribute__((always_inline)) {
    if (copy) slab_ops(jj + F8_NST, ops);
    load_frags(jj + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    mma(cur, copy ? &ops : nullptr);
    __builtin_amdgcn_sched_barrier(0);
    if (copy) __builtin_amdgcn_s_waitcnt(F8_VMCNT((F8_NST - 2) * F8_OPS));
    else f8_wait_slabs<F8_OPS>(nk - 1 - (jj + 2));
    __syncthreads();
  };
  // the main loop runs intervals in pairs so the two fragment sets swap roles
  // without register copies
  int j = 0;
  for (; j + 1 + F8_NST < nk; j += 2) {
    interval(j, f0, f1, true);
    interval(j + 1, f1, f0, true);
  }
  // Interval j always works on f0 for even j and f1 for odd j.  After the
  // pairs, at most one interval still copies (j + NST == nk - 1); at most
  // NST - 1 intervals are left in all, drained as one pair and one single;
  // the last slab's MFMAs close.
  if (j + F8_NST < nk) {
    interval(j, f0, f1, true);
    interval(j + 1, f1, f0, false);
    j += 2;
  }
  if (j + 2 < nk) {  // at most once: at most NST - 1 = 3 intervals are left here
    interval(j, f0, f1, false);
    interval(j + 1, f1, f0, false);
    j += 2;
  }
  if (j + 1 < nk) {
    interval(j, f0, f1, false);
    mma(f1, nullptr);
  } else {
    mma(f0, nullptr);
  }
#undef F8_COPY

  if (p.c_f32) {
    float *C = reinterpret_cast<float *>(p.c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = n0 + wn * 128 + jj * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 128 + i * 32 + acc_row(r, lane);
          if (m < p.M && n < p.N) C[(int64_t)m * p.ldc + n] = acc[i][jj][r];
        }
      }
    return;
  }
  // bf16: through LDS (the stages are free after the last barrier), then
  // 16-byte row runs
  __syncthreads();
  bf16 *Cs = reinterpret_cast<bf16 *>(lds);
  if (p.nseg > 0 && F8_SEG(p, f8_seg_of(p, min(n0, p.N - 1)), tr)) {
    // channel-major column range (aligned to the tile on the host): the tile
    // goes to LDS transposed, a lane writing its four consecutive rows of a
    // column as one 8-byte store; then lanes take 8-token runs of a column
    constexpr int TP = F8_BM + 8;
    static_assert(F8_BN * TP * 2 <= F8_LDS, "transposed tile must fit the LDS area");
    const int st0 = f8_seg_of(p, min(n0, p.N - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16 v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)acc[i][jj][4 * q + e];
          *reinterpret_cast<uint2 *>(&Cs[(wn * 128 + jj * 32 + l32) * TP + wm * 128 + i * 32 +
                                         acc_row(4 * q, lane)]) = *reinterpret_cast<const uint2 *>(v4);
        }
    __syncthreads();
    bf16 *t_C = reinterpret_cast<bf16 *>(F8_SEG(p, st0, C));
    const int t_dh = F8_SEG(p, st0, dh), t_nb = F8_SEG(p, st0, n_begin);
    constexpr int RG = F8_BM / 8;  // 8-token runs per column
    for (int it = 0; it < (F8_BM * F8_BN / 8) / F8_THREADS; ++it) {
      const int c = tid + F8_THREADS * it;
      const int col = c / RG, rg = c - col * RG;
      const int m = m0 + rg * 8, n = n0 + col;
      if (m >= p.M || n >= p.N) continue;
      const int nn = n - t_nb;
      const int h = nn / t_dh, d = nn - h * t_dh;
      const int b = m / p.S, sq = m - b * p.S;
      const bf16 *src = &Cs[col * TP + rg * 8];
      if (sq + 8 <= p.S && m + 8 <= p.M) {
        *reinterpret_cast<uint4 *>(t_C + ((int64_t)(b * p.H + h) * t_dh + d) * p.S + sq) =
            *reinterpret_cast<const uint4 *>(src);
      } else {
        for (int e = 0; e < 8 && m + e < p.M; ++e) {
          const int me = m + e, be = me / p.S, se = me - be * p.S;
          t_C[((int64_t)(be * p.H + h) * t_dh + d) * p.S + se] = src[e];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Cs[(wm * 128 + i * 32 + acc_row(r, lane)) * F8_CPITCH + wn * 128 + jj * 32 + l32] = (bf16)acc[i][jj][r];
  __syncthreads();
  bf16 *C = reinterpret_cast<bf16 *>(p.c);
  constexpr int RUNS = F8_BN / 8;
  for (int it = 0; it < (F8_BM * RUNS) / F8_THREADS; ++it) {
    const int c = tid + F8_THREADS * it;
    const int row = c / RUNS, cc = c - row * RUNS;
    const int m = m0 + row, n = n0 + cc * 8;
    if (m >= p.M || n >= p.N) continue;
    bf16 *dst = C + (int64_t)m * p.ldc + n;
    if (p.nseg > 0) {
      // head-major scatter: a run of 8 columns lies in one head of one range
      const int s = f8_seg_of(p, n);
      const int nn = n - F8_SEG(p, s, n_begin), dh = F8_SEG(p, s, dh);
      const int h = nn / dh, d = nn - h * dh;
      const int b = m / p.S, sq = m - b * p.S;
      dst = reinterpret_cast<bf16 *>(F8_SEG(p, s, C)) +
            ((int64_t)(b * p.H + h) * p.S + sq) * F8_SEG(p, s, ld) + F8_SEG(p, s, off) + d;
    }
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(&Cs[row * F8_CPITCH + cc * 8]);
  }
}

// E8M0 exponent of a tile: the smallest e with amax <= 448 * 2^e (448 =
// 0.875 * 2^9, so from amax = f 2^E, f in [0.5, 1): e = E - 9 + (f > 0.875)),
// 0 for an all-zero tile, clamped to [-127, 127].
__device__ inline int f8_tile_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = E - 9 + (f > 0.875f ? 1 : 0);
  return min(max(e, -127), 127);
}

template <typename T> __device__ inline float f8_ld(const T *p) { return (float)*p; }

// 1 x 128 activation tiles: a wave takes four consecutive tiles of a row,
// 16 lanes per tile and 8 consecutive values per lane (16-byte loads and
// 8-byte code stores when `vec`; element accesses otherwise).
template <typename T>
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const T *x, int64_t rows, int64_t ldx, int tiles,
                                                             uint8_t *q, int64_t ldq, uint8_t *sexp,
                                                             int64_t lds_, int vec) {
  const int groups = (tiles + 3) / 4;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= rows * groups) return;
  const int64_t row = w / groups;
  const int kb = (int)(w - row * groups) * 4 + (lane >> 4);
  const bool live = kb < tiles;
  const int64_t col = (int64_t)kb * F8_TILE + 8 * (lane & 15);
  float v[8];
  if (live && vec) {
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4 *>(x + row * ldx + col);
      const bf16 *h = reinterpret_cast<const bf16 *>(&u);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
    } else {
      const float4 u0 = *reinterpret_cast<const float4 *>(x + row * ldx + col);
      const float4 u1 = *reinterpret_cast<const float4 *>(x + row * ldx + col + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = live ? f8_ld(x + row * ldx + col + i) : 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));   // within the 16-lane tile
  const int e = f8_tile_exponent(amax);
  uint32_t pk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * i], -e), ldexpf(v[4 * i + 1], -e), 0, false);
    pk[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * i + 2], -e), ldexpf(v[4 * i + 3], -e), lo, true);
  }
  if (!live) return;
  uint8_t *dst = q + row * ldq + col;
  if (vec) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(pk[0], pk[1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<uint16_t *>(dst)[i] = (uint16_t)(pk[i >> 1] >> (16 * (i & 1)));
  }
  if ((lane & 15) == 0) sexp[(int64_t)kb * lds_ + row] = (uint8_t)(e + 127);
}

// 128 x 128 weight blocks: one workgroup per block, thread t takes row t / 2
// of the block and 64 consecutive columns; every row of the block gets the
// block's exponent byte.
template <typename T>
__global__ __launch_bounds__(256) void fp8_quant_blocks_kernel(const T *w, int64_t rows, int64_t ldw, uint8_t *q,
                                                               int64_t ldq, uint8_t *sexp, int64_t lds_) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * F8_TILE + (tid >> 1);
  const int kb = blockIdx.y;
  const int c0 = kb * F8_TILE + (tid & 1) * 64;
  const bool live = r < rows;
  float v[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) v[i] = live ? f8_ld(w + r * ldw + c0 + i) : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = f8_tile_exponent(amax);
  if (!live) return;
  uint32_t packed[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * i], -e), ldexpf(v[4 * i + 1], -e), 0, false);
    packed[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * i + 2], -e), ldexpf(v[4 * i + 3], -e), lo,
                                                          true);
  }
  uint4 *dst = reinterpret_cast<uint4 *>(q + r * ldq + c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(packed[4 * i], packed[4 * i + 1], packed[4 * i + 2], packed[4 * i + 3]);
  if ((tid & 1) == 0) sexp[(int64_t)kb * lds_ + r] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_fp8_quant_rows(int dtype, const void *x, int64_t rows, int64_t cols, int64_t ldx, uint8_t *q,
                                 int64_t ldq, uint8_t *sexp, int64_t ld_s, hipStream_t st) {
  const int tiles = (int)(cols / F8_TILE);
  const int64_t waves = rows * ((tiles + 3) / 4);
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  const size_t es = dtype == BF16 ? 2 : 4;
  const int vec = ((uintptr_t)x % 16 == 0 && (ldx * es) % 16 == 0 && (uintptr_t)q % 8 == 0 && ldq % 8 == 0) ? 1 : 0;
  if (dtype == BF16)
    hipLaunchKernelGGL(fp8_quant_rows_kernel<bf16>, grid, dim3(256), 0, st, reinterpret_cast<const bf16 *>(x), rows,
                       ldx, tiles, q, ldq, sexp, ld_s, vec);
  else
    hipLaunchKernelGGL(fp8_quant_rows_kernel<float>, grid, dim3(256), 0, st, reinterpret_cast<const float *>(x),
                       rows, ldx, tiles, q, ldq, sexp, ld_s, vec);
  return hipGetLastError();
}

hipError_t launch_fp8_quant_blocks(int dtype, const void *w, int64_t rows, int64_t cols, int64_t ldw, uint8_t *q,
                                   int64_t ldq, uint8_t *sexp, int64_t ld_s, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + F8_TILE - 1) / F8_TILE), (unsigned)(cols / F8_TILE));
  if (dtype == BF16)
    hipLaunchKernelGGL(fp8_quant_blocks_kernel<bf16>, grid, dim3(256), 0, st, reinterpret_cast<const bf16 *>(w),
                       rows, ldw, q, ldq, sexp, ld_s);
  else
    hipLaunchKernelGGL(fp8_quant_blocks_kernel<float>, grid, dim3(256), 0, st, reinterpret_cast<const float *>(w),
                       rows, ldw, q, ldq, sexp, ld_s);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa, const uint8_t *b,
                           int64_t ldb, const uint8_t *sb, int64_t ld_sb, void *c, int c_dtype, int64_t ldc, int M,
                           int N, int K, hipStream_t st) {
  if (M == 0) return hipSuccess;
  Fp8GemmParams p{a, sa, b, sb, lda, ld_sa, ldb, ld_sb, ldc, c, M, N, K, c_dtype == F32 ? 1 : 0};
  const int tm = (M + F8_BM - 1) / F8_BM, tn = (N + F8_BN - 1) / F8_BN;
  const int T = tm * tn;
  const int group_m = K >= 8192 ? 8 : (K <= 2048 ? 2 : 4);
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3(T), dim3(F8_THREADS), 0, st, p, tm, tn, (T % 8 == 0) ? 1 : 0,
                     group_m);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm_seg(const Fp8GemmDesc &d, hipStream_t st) {
  if (d.M == 0) return hipSuccess;
  Fp8GemmParams p{d.a, d.sa, d.b, d.sb, d.lda, d.ld_sa, d.ldb, d.ld_sb, 0, nullptr, d.M, d.N, d.K, 0};
  p.S = d.S;
  p.H = d.H;
  p.nseg = d.nseg;
  for (int s = 0; s < 3; ++s) p.seg[s] = d.seg[s];
  const int tm = (d.M + F8_BM - 1) / F8_BM, tn = (d.N + F8_BN - 1) / F8_BN;
  const int T = tm * tn;
  const int group_m = d.K >= 8192 ? 8 : (d.K <= 2048 ? 2 : 4);
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3(T), dim3(F8_THREADS), 0, st, p, tm, tn, (T % 8 == 0) ? 1 : 0,
                     group_m);
  return hipGetLastError();
}

int64_t fp8_scale_pitch(int64_t rows) { return (rows + F8_BM - 1) / F8_BM * F8_BM; }

}  // namespace mla
