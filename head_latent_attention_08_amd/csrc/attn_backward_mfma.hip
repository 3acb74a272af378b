// Causal attention backward on the matrix cores (gfx950, bf16).
//
// The gradients of O = softmax(scale Q K^T, tril) V per head (the forward of
// "The Evolving Transformer -- DeepSeek V2 & V3", section 01):
//   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale dS K,
//   dK = scale dS^T Q,
// with P recomputed from each query's log-sum-exp.  Three passes, each a
// workgroup of four waves over a 128-row block of one head, every product on
// 32x32x16 bf16 MFMAs with fp32 accumulation, and no atomics (every sum runs
// in a fixed order, so the result is deterministic):
//
// * row statistics: per query, lse (log2 domain, from S^T = K Q^T over its
//   keys with an online max) and delta = rowsum(dO * O), stored interleaved
//   as one float2 per row;
// * dK, dV: a wave owns 32 keys (their K and V rows stay in registers as the
//   B operands of S = Q K^T and dP = dO V^T) and walks the query tiles at and
//   after its keys.  S's accumulators hold one key column per lane, so P and
//   dS feed dV += P^T dO and dK += dS^T Q straight from the accumulators as
//   the A operand; the matching dO / Q operand (8 queries of one channel per
//   lane) comes from the row-major tile in LDS through the 16-bit transposing
//   LDS read;
// * dQ: a wave owns 32 queries (Q and dO rows in registers) and walks the key
//   tiles up to its queries; S^T = K Q^T holds one query column per lane, so
//   dS feeds dQ += dS K the same way, K's operand through the transposing
//   read.
//
// Tiles of 32 rows stream global -> LDS with global_load_lds_dwordx4 (no
// staging registers) through three stages, two tiles ahead, one barrier per
// tile.  A tile is stored unpadded, 16-byte chunks XOR-permuted per row (see
// tile_swz), so both the row-fragment reads (16 rows, one chunk) and the
// transposing reads (4 rows, 4 chunks) of a quarter wave hit distinct banks.
// Rows past the sequence repeat the last row (finite data that the masks
// drop).

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int BT = 32;        // rows per tile
constexpr int BW = 4;         // waves per workgroup
constexpr int BROWS = BT * BW;
constexpr float BLOG2E = 1.4426950408889634f;

typedef short s16x4b __attribute__((ext_vector_type(4)));

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (gfx9 encoding; expcnt and lgkmcnt left open)
#define BWD_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Wait until at most n (uniform, 0..8) of this wave's copies are in flight.
__device__ inline void wait_copies(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(7)); break;
    default: __builtin_amdgcn_s_waitcnt(BWD_VMCNT(8)); break;
  }
}

template <typename P> __device__ inline P *wave_uniform(P *q) {
  const uint64_t v = (uint64_t)q;
  return reinterpret_cast<P *>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                               (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}

// A 32-row tile of W bf16 columns in LDS: rows of 2W bytes, no padding, the
// 16-byte chunk c of row r at position c ^ tile_swz(r).  The permutation
// keeps a chunk inside its aligned group of 8 (4 for W = 96), so it stays in
// the row.  Row-fragment reads: 16 consecutive rows, one chunk; transposing
// reads: 4 consecutive rows (aligned to 4), 4 chunks (aligned to 4).  With
// 2W/16 chunks per row:
//  * = 8 mod 16 (W = 192, 64): consecutive rows alternate halves of the 16
//    bank groups; the swizzle permutes (r / 2) % 8 so that rows r and r + 2
//    land in different 4-chunk groups;
//  * = 0 mod 16 (W = 128): all rows start in bank group 0; the swizzle is a
//    permutation of r % 16 whose upper two bits differ within every 4 rows;
//  * = 12 (W = 96): rows start 12 groups apart, so 4 consecutive rows are
//    already distinct; rows 4 apart get (r / 4) % 4.
template <int W> __device__ inline int tile_swz(int r) {
  if constexpr ((W / 8) % 16 == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else if constexpr ((W / 8) % 16 == 0) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

template <int W> struct Tile {
  static_assert(W == 192 || W == 128 || W == 96 || W == 64, "tile width");
  static constexpr int ROWB = 2 * W;
  static constexpr int BYTES = BT * ROWB;   // 64 W: W / 16 whole 1 KB copy blocks
  static constexpr int NBLK = BYTES / 1024;
  static constexpr int NPW = (NBLK + BW - 1) / BW;  // copy blocks per wave (at most)
};

// A wave's share of one tile's copies: blocks wave, wave + 4, ..; lane l of
// block b fills LDS bytes 1024 b + 16 l, i.e. row r = (1024 b + 16 l) / 2W at
// chunk position p, which holds logical chunk p ^ tile_swz(r).
template <int W> struct TileCopy {
  using TL = Tile<W>;
  int row[TL::NPW], cb[TL::NPW];  // tile row and byte column in the source row
  int n;                          // copy instructions this wave issues per tile
  __device__ void init(int wave, int lane) {
    n = 0;
#pragma unroll
    for (int k = 0; k < TL::NPW; ++k) {
      const int b = wave + BW * k;
      const int o = b * 1024 + lane * 16, r = o / TL::ROWB, p = (o - r * TL::ROWB) / 16;
      row[k] = b < TL::NBLK ? r : 0;
      cb[k] = b < TL::NBLK ? 16 * (p ^ tile_swz<W>(r)) : 0;
      n += b < TL::NBLK ? 1 : 0;
    }
  }
  // tile of rows r0 .. r0 + 31 of base ([rows, W] row-major) into LDS at lds
  __device__ void issue(const bf16 *base, int r0, int rows, uint32_t lds, int wave) const {
    const bf16 *tb = wave_uniform(base + (int64_t)r0 * W);
    const int lim = rows - 1 - r0;
#pragma unroll
    for (int k = 0; k < TL::NPW; ++k) {
      const int b = wave + BW * k;
      if (b < TL::NBLK) {
        const uint32_t off = (uint32_t)(min(row[k], lim) * TL::ROWB + cb[k]);
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds + b * 1024);
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(tb), "s"(m0) : "memory", "m0");
      }
    }
  }
};

// A / B fragment of a 32x32x16 step from a tile: row l32, logical chunk
// 2 f + g (channels 16 f + 8 g .. + 7).
template <int W>
__device__ inline bf16x8 row_frag(const char *t, int l32, int g, int f) {
  return *reinterpret_cast<const bf16x8 *>(t + l32 * Tile<W>::ROWB + 16 * ((2 * f + g) ^ tile_swz<W>(l32)));
}

// B fragment whose k values are tile rows: lane (column 32 d + l32, half g)
// receives rows 16 u + 4 g + 0..3 and 16 u + 8 + 4 g + 0..3 of its column,
// the row order of the accumulator rows 8 u .. 8 u + 7 (acc_row).  Two
// transposing reads: within a 16-lane group lane i gets element i % 4 of the
// 8-byte pieces of lanes 4 e + i / 4, so lane s reads row 16 u + 4 g + s / 4,
// columns 32 d + (lane & 16) + 4 (s % 4) .. + 3.
template <int W>
__device__ inline bf16x8 col_frag(const char *t, int lane, int u, int d) {
  const int s16 = lane & 15, g = lane >> 5;
  const int c = 4 * d + ((lane >> 4) & 1) * 2 + ((s16 & 3) >> 1), h = 8 * (s16 & 1);
  const int r0 = 16 * u + 4 * g + (s16 >> 2), r1 = r0 + 8;
  const char *p0 = t + r0 * Tile<W>::ROWB + 16 * (c ^ tile_swz<W>(r0)) + h;
  const char *p1 = t + r1 * Tile<W>::ROWB + 16 * (c ^ tile_swz<W>(r1)) + h;
  const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4b *)p0);
  const s16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4b *)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline bf16x8 pack8(const f32x16 &a, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)a[8 * u + e];
  return r;
}

__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// Workgroup -> (head, block): the blocks of a head run on one XCD
// (workgroup ids go to the eight XCDs round-robin), longest blocks first; an
// XCD takes its heads two at a time with their blocks interleaved, so the
// long blocks of the last heads do not start at the end.
__device__ inline void block_of(int BH, int nb, int &bh, int &blk, bool reverse) {
  const int w = blockIdx.x;
  if ((BH & 15) == 0) {
    const int local = w >> 3;
    const int grp = local / (2 * nb), r = local - grp * (2 * nb);
    bh = (w & 7) * (BH >> 3) + 2 * grp + (r & 1);
    blk = r >> 1;
  } else if ((BH & 7) == 0) {
    const int local = w >> 3;
    bh = (w & 7) * (BH >> 3) + local / nb;
    blk = local % nb;
  } else {
    bh = w / nb;
    blk = w % nb;
  }
  if (reverse) blk = nb - 1 - blk;
}

// ---------------------------------------------------------- row statistics
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_stats_kernel(AttnBwdArgs a) {
  constexpr int NQF = DQK / 16;
  using TK = Tile<DQK>;
  __shared__ __attribute__((aligned(1024))) char Ks[3][TK::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, nb = (S + BROWS - 1) / BROWS;
  int bh, blk;
  block_of(a.BH, nb, bh, blk, true);
  const bf16 *q = reinterpret_cast<const bf16 *>(a.q) + (int64_t)bh * S * DQK;
  const bf16 *k = reinterpret_cast<const bf16 *>(a.k) + (int64_t)bh * S * DQK;
  const int q0 = blk * BROWS, qw = q0 + wave * BT, qi = qw + l32;
  bf16x8 qf[NQF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    qf[f] = bf16x8{};
    if (qi < S) qf[f] = *reinterpret_cast<const bf16x8 *>(q + (int64_t)qi * DQK + 16 * f + 8 * g);
  }
  const float sl2 = a.scale * BLOG2E;
  float m = -INFINITY, l = 0.f;
  const int ntiles = (min(S, q0 + BROWS) + BT - 1) / BT;
  const int last = qw / BT;  // this wave's diagonal tile
  TileCopy<DQK> ck;
  ck.init(wave, lane);
  const uint32_t kl = lds_addr(Ks);
  ck.issue(k, 0, S, kl, wave);
  if (ntiles > 1) ck.issue(k, BT, S, kl + TK::BYTES, wave);
  wait_copies(ntiles > 1 ? ck.n : 0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 2 < ntiles) ck.issue(k, (t + 2) * BT, S, kl + ((t + 2) % 3) * TK::BYTES, wave);
    if (t <= last) {
      const char *kt = Ks[t % 3];
      f32x16 s = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<DQK>(kt, l32, g, f), qf[f], s, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t * BT + acc_row(r, lane);
        if (kj > qi) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      const float mn = fmaxf(m, mx);
      if (mn != -INFINITY) {
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f((s[r] - mn) * sl2);
        l = l * __builtin_amdgcn_exp2f((m - mn) * sl2) + sum;
        m = mn;
      }
    }
    wait_copies(t + 2 < ntiles ? ck.n : 0);
    __syncthreads();
  }
  // the two halves of the wave hold the same query's rows
  const float M = half_swap_max(m);
  const float lw = (m == -INFINITY) ? 0.f : l * __builtin_amdgcn_exp2f((m - M) * sl2);
  const float L = half_swap_sum(lw);
  // delta = rowsum(dO * O): half g takes channels [g DV/2, (g+1) DV/2)
  float dl = 0.f;
  if (qi < S) {
    const bf16 *o = reinterpret_cast<const bf16 *>(a.o) + ((int64_t)bh * S + qi) * DV + g * (DV / 2);
    const bf16 *dout = reinterpret_cast<const bf16 *>(a.dout) + ((int64_t)bh * S + qi) * DV + g * (DV / 2);
#pragma unroll
    for (int c = 0; c < DV / 2; c += 8) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8 *>(o + c), dv = *reinterpret_cast<const bf16x8 *>(dout + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = fmaf((float)ov[e], (float)dv[e], dl);
    }
  }
  dl = half_swap_sum(dl);
  if (qi < S && g == 0) {
    // log2 domain: P = exp2(s sl2 - lse)
    reinterpret_cast<float2 *>(a.lse)[(int64_t)bh * S + qi] = make_float2(M * sl2 + __builtin_amdgcn_logf(L), dl);
  }
}

// ------------------------------------------------------------------ dK, dV
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int NQF = DQK / 16, NVF = DV / 16, NKT = DQK / 32, NVT = DV / 32;
  using TQ = Tile<DQK>;
  using TV = Tile<DV>;
  __shared__ __attribute__((aligned(1024))) char Qs[3][TQ::BYTES];
  __shared__ __attribute__((aligned(1024))) char Os[3][TV::BYTES];  // dO tiles
  __shared__ __attribute__((aligned(16))) float2 St[3][BT];         // (lse, delta) of the tile's queries
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, nb = (S + BROWS - 1) / BROWS;
  int bh, blk;
  block_of(a.BH, nb, bh, blk, false);  // early key blocks see the most queries
  const int64_t hoff = (int64_t)bh * S;
  const bf16 *q = reinterpret_cast<const bf16 *>(a.q) + hoff * DQK;
  const bf16 *k = reinterpret_cast<const bf16 *>(a.k) + hoff * DQK;
  const bf16 *v = reinterpret_cast<const bf16 *>(a.v) + hoff * DV;
  const bf16 *dout = reinterpret_cast<const bf16 *>(a.dout) + hoff * DV;
  const float *stats = a.lse + 2 * hoff;
  const int k0 = blk * BROWS, kw = k0 + wave * BT, kj = kw + l32;  // this lane's key
  bf16x8 kf[NQF], vf[NVF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    kf[f] = bf16x8{};
    if (kj < S) kf[f] = *reinterpret_cast<const bf16x8 *>(k + (int64_t)kj * DQK + 16 * f + 8 * g);
  }
#pragma unroll
  for (int f = 0; f < NVF; ++f) {
    vf[f] = bf16x8{};
    if (kj < S) vf[f] = *reinterpret_cast<const bf16x8 *>(v + (int64_t)kj * DV + 16 * f + 8 * g);
  }
  f32x16 dk[NKT], dv[NVT];
#pragma unroll
  for (int d = 0; d < NKT; ++d) dk[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < NVT; ++d) dv[d] = f32x16{};
  const float sl2 = a.scale * BLOG2E;
  const int t0 = k0 / BT, ntiles = (S + BT - 1) / BT;
  TileCopy<DQK> cq;
  TileCopy<DV> co;
  cq.init(wave, lane);
  co.init(wave, lane);
  // the last wave also copies the tile's 32 (lse, delta) pairs: 256 bytes,
  // lane l the 4 bytes at 4 l (rows past the sequence repeat the last row)
  const bool stat_wave = wave == BW - 1;
  const int ncp = cq.n + co.n + (stat_wave ? 1 : 0);
  const uint32_t ql = lds_addr(Qs), ol = lds_addr(Os), sl = lds_addr(St);
  auto issue = [&](int t) {
    const int st = t % 3;
    cq.issue(q, t * BT, S, ql + st * TQ::BYTES, wave);
    co.issue(dout, t * BT, S, ol + st * TV::BYTES, wave);
    if (stat_wave) {
      const float *sb = wave_uniform(stats + 2 * (int64_t)t * BT);
      const uint32_t off = (uint32_t)(min(lane >> 1, S - 1 - t * BT) * 8 + 4 * (lane & 1));
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(sl + st * BT * 8);
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                   :: "v"(off), "s"(sb), "s"(m0) : "memory", "m0");
    }
  };
  issue(t0);
  if (t0 + 1 < ntiles) issue(t0 + 1);
  wait_copies(t0 + 1 < ntiles ? ncp : 0);
  __syncthreads();
  for (int t = t0; t < ntiles; ++t) {
    if (t + 2 < ntiles) issue(t + 2);
    // queries of tile t that this wave's keys can see: qi >= kj for some lane
    if (t * BT + BT - 1 >= kw) {
      const int st = t % 3;
      const char *qt = Qs[st], *ot = Os[st];
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<DQK>(qt, l32, g, f), kf[f], s, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NVF; ++f)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<DV>(ot, l32, g, f), vf[f], dp, 0, 0, 0);
      // P and dS: row r is query t BT + acc_row(r), the lane's column key kj
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = acc_row(r, lane), qi = t * BT + qr;
        const float2 ld = St[st][qr];
        const float p = (kj <= qi && qi < S) ? __builtin_amdgcn_exp2f(s[r] * sl2 - ld.x) : 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - ld.y);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pa = pack8(s, u), da = pack8(dp, u);
#pragma unroll
        for (int d = 0; d < NVT; ++d)
          dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, col_frag<DV>(ot, lane, u, d), dv[d], 0, 0, 0);
#pragma unroll
        for (int d = 0; d < NKT; ++d)
          dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, col_frag<DQK>(qt, lane, u, d), dk[d], 0, 0, 0);
      }
    }
    wait_copies(t + 2 < ntiles ? ncp : 0);
    __syncthreads();
  }
  // accumulator (r, lane): key kw + acc_row(r), channel 32 d + l32
  bf16 *dkp = reinterpret_cast<bf16 *>(a.dk) + hoff * DQK;
  bf16 *dvp = reinterpret_cast<bf16 *>(a.dvo) + hoff * DV;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kw + acc_row(r, lane);
    if (key < S) {
#pragma unroll
      for (int d = 0; d < NKT; ++d) dkp[(int64_t)key * DQK + 32 * d + l32] = (bf16)(a.scale * dk[d][r]);
#pragma unroll
      for (int d = 0; d < NVT; ++d) dvp[(int64_t)key * DV + 32 * d + l32] = (bf16)dv[d][r];
    }
  }
}

// --------------------------------------------------------------------- dQ
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int NQF = DQK / 16, NVF = DV / 16, NKT = DQK / 32;
  using TK = Tile<DQK>;
  using TV = Tile<DV>;
  __shared__ __attribute__((aligned(1024))) char Ks[3][TK::BYTES];
  __shared__ __attribute__((aligned(1024))) char Vs[3][TV::BYTES];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, nb = (S + BROWS - 1) / BROWS;
  int bh, blk;
  block_of(a.BH, nb, bh, blk, true);
  const int64_t hoff = (int64_t)bh * S;
  const bf16 *q = reinterpret_cast<const bf16 *>(a.q) + hoff * DQK;
  const bf16 *k = reinterpret_cast<const bf16 *>(a.k) + hoff * DQK;
  const bf16 *v = reinterpret_cast<const bf16 *>(a.v) + hoff * DV;
  const bf16 *dout = reinterpret_cast<const bf16 *>(a.dout) + hoff * DV;
  const int q0 = blk * BROWS, qw = q0 + wave * BT, qi = qw + l32;  // this lane's query
  bf16x8 qf[NQF], of[NVF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    qf[f] = bf16x8{};
    if (qi < S) qf[f] = *reinterpret_cast<const bf16x8 *>(q + (int64_t)qi * DQK + 16 * f + 8 * g);
  }
#pragma unroll
  for (int f = 0; f < NVF; ++f) {
    of[f] = bf16x8{};
    if (qi < S) of[f] = *reinterpret_cast<const bf16x8 *>(dout + (int64_t)qi * DV + 16 * f + 8 * g);
  }
  const float2 ld = qi < S ? reinterpret_cast<const float2 *>(a.lse)[hoff + qi] : make_float2(0.f, 0.f);
  f32x16 dq[NKT];
#pragma unroll
  for (int d = 0; d < NKT; ++d) dq[d] = f32x16{};
  const float sl2 = a.scale * BLOG2E;
  const int ntiles = (min(S, q0 + BROWS) + BT - 1) / BT;
  const int last = qw / BT;  // this wave's diagonal tile
  TileCopy<DQK> ck;
  TileCopy<DV> cv;
  ck.init(wave, lane);
  cv.init(wave, lane);
  const int ncp = ck.n + cv.n;
  const uint32_t kl = lds_addr(Ks), vl = lds_addr(Vs);
  auto issue = [&](int t) {
    const int st = t % 3;
    ck.issue(k, t * BT, S, kl + st * TK::BYTES, wave);
    cv.issue(v, t * BT, S, vl + st * TV::BYTES, wave);
  };
  issue(0);
  if (ntiles > 1) issue(1);
  wait_copies(ntiles > 1 ? ncp : 0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 2 < ntiles) issue(t + 2);
    if (t <= last) {
      const int st = t % 3;
      const char *kt = Ks[st], *vt = Vs[st];
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<DQK>(kt, l32, g, f), qf[f], s, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NVF; ++f)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<DV>(vt, l32, g, f), of[f], dp, 0, 0, 0);
      // row r is key t BT + acc_row(r), the lane's column query qi
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t * BT + acc_row(r, lane);
        const float p = (kj <= qi && qi < S) ? __builtin_amdgcn_exp2f(s[r] * sl2 - ld.x) : 0.f;
        dp[r] = p * (dp[r] - ld.y);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 da = pack8(dp, u);
#pragma unroll
        for (int d = 0; d < NKT; ++d)
          dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, col_frag<DQK>(kt, lane, u, d), dq[d], 0, 0, 0);
      }
    }
    wait_copies(t + 2 < ntiles ? ncp : 0);
    __syncthreads();
  }
  // accumulator (r, lane): query qw + acc_row(r), channel 32 d + l32
  bf16 *dqp = reinterpret_cast<bf16 *>(a.dq) + hoff * DQK;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qq = qw + acc_row(r, lane);
    if (qq < S) {
#pragma unroll
      for (int d = 0; d < NKT; ++d) dqp[(int64_t)qq * DQK + 32 * d + l32] = (bf16)(a.scale * dq[d][r]);
    }
  }
}

template <int DQK, int DV> hipError_t launch_mfma_t(const AttnBwdArgs &a, hipStream_t st) {
  const int nb = (a.S + BROWS - 1) / BROWS;
  const dim3 grid((unsigned)((int64_t)a.BH * nb)), block(256);
  hipLaunchKernelGGL((bwd_stats_kernel<DQK, DV>), grid, block, 0, st, a);
  hipLaunchKernelGGL((bwd_dkdv_kernel<DQK, DV>), grid, block, 0, st, a);
  hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool attention_backward_mfma_supported(int dtype, int dqk, int dv) {
  return dtype == BF16 && ((dqk == 192 && dv == 128) || (dqk == 96 && dv == 64) || (dqk == 64 && dv == 64));
}

hipError_t launch_attention_backward_mfma(const AttnBwdArgs &a, hipStream_t st) {
  if ((int64_t)a.BH * a.S == 0) return hipSuccess;
  if (a.dqk == 192 && a.dv == 128) return launch_mfma_t<192, 128>(a, st);
  if (a.dqk == 96 && a.dv == 64) return launch_mfma_t<96, 64>(a, st);
  if (a.dqk == 64 && a.dv == 64) return launch_mfma_t<64, 64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace mla
