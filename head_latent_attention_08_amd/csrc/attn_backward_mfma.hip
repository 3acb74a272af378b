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
//   keys with an online max) and delta = rowsum(dO * O);
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
// Tiles of 32 rows are double-buffered in LDS: the next tile is loaded into
// registers while the current one is computed, stored after, one barrier per
// tile.  Rows past the sequence load as zeros and are masked.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int BT = 32;        // rows per tile
constexpr int BW = 4;         // waves per workgroup
constexpr int BROWS = BT * BW;
constexpr float BLOG2E = 1.4426950408889634f;

typedef short s16x4b __attribute__((ext_vector_type(4)));

template <int W> struct TileLds {
  static constexpr int PITCH = W + 8;             // elements (16 B of padding)
  static constexpr int ELEMS = BT * PITCH;
  static constexpr int CHUNKS = BT * W / 8;       // 16-byte chunks per tile
};

// 16-byte chunks of rows r0.. of a [rows, W] bf16 matrix into registers
// (zeros past `rows`); chunk c = tid + 256 i.
template <int W, int NCH>
__device__ inline void load_tile(const bf16 *base, int r0, int rows, int tid, uint4 (&v)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (c < TileLds<W>::CHUNKS) {
      const int r = c / (W / 8), cc = (c - r * (W / 8)) * 8;
      if (r0 + r < rows) v[i] = *reinterpret_cast<const uint4 *>(base + (int64_t)(r0 + r) * W + cc);
    }
  }
}

template <int W, int NCH>
__device__ inline void store_tile(bf16 *lds, int tid, const uint4 (&v)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    if (c < TileLds<W>::CHUNKS) {
      const int r = c / (W / 8), cc = (c - r * (W / 8)) * 8;
      *reinterpret_cast<uint4 *>(lds + r * TileLds<W>::PITCH + cc) = v[i];
    }
  }
}

// A / B fragment of a 32x32x16 step from a row-major LDS tile: row l32,
// channels 16 f + 8 g .. + 7.
template <int PITCH>
__device__ inline bf16x8 row_frag(const bf16 *t, int l32, int g, int f) {
  return *reinterpret_cast<const bf16x8 *>(t + l32 * PITCH + 16 * f + 8 * g);
}

// B fragment whose k values are tile rows: lane (column 32 d + l32, half g)
// receives rows 16 u + 4 g + 0..3 and 16 u + 8 + 4 g + 0..3 of its column,
// the row order of the accumulator rows 8 u .. 8 u + 7 (acc_row).  Two
// transposing reads: within a 16-lane group lane i gets element i % 4 of the
// 8-byte chunks of lanes 4 e + i / 4, so lane s points at row
// 16 u + 4 g + s / 4, column 32 d + (lane & 16) + 4 (s % 4).
template <int PITCH>
__device__ inline bf16x8 col_frag(const bf16 *t, int lane, int u, int d) {
  const int s16 = lane & 15, g = lane >> 5;
  const bf16 *p = t + (16 * u + 4 * g + (s16 >> 2)) * PITCH + 32 * d + (lane & 16) + 4 * (s16 & 3);
  const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4b *)p);
  const s16x4b hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4b *)(p + 8 * PITCH));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline bf16x8 pack8(const f32x16 &a, int u) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)a[8 * u + e];
  return r;
}

// Workgroup -> (head, block): the blocks of a head run on one XCD
// (workgroup ids go to the eight XCDs round-robin), longest blocks first.
__device__ inline void block_of(int BH, int nb, int &bh, int &blk, bool reverse) {
  const int w = blockIdx.x;
  if ((BH & 7) == 0) {
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
  using TK = TileLds<DQK>;
  constexpr int NCK = (TK::CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TK::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
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
  const int last = (qw + BT - 1) / BT;  // this wave's last key tile
  uint4 rk[NCK];
  load_tile<DQK, NCK>(k, 0, S, tid, rk);
  store_tile<DQK, NCK>(Ks[0], tid, rk);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile<DQK, NCK>(k, (t + 1) * BT, S, tid, rk);
    if (t <= last) {
      const bf16 *kt = Ks[t & 1];
      f32x16 s = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<TK::PITCH>(kt, l32, g, f), qf[f], s, 0, 0, 0);
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
    if (t + 1 < ntiles) store_tile<DQK, NCK>(Ks[(t + 1) & 1], tid, rk);
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
    a.lse[(int64_t)bh * S + qi] = M * sl2 + __builtin_amdgcn_logf(L);  // log2 domain: exp2(s sl2 - lse)
    a.delta[(int64_t)bh * S + qi] = dl;
  }
}

// ------------------------------------------------------------------ dK, dV
template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int NQF = DQK / 16, NVF = DV / 16, NKT = DQK / 32, NVT = DV / 32;
  using TQ = TileLds<DQK>;
  using TV = TileLds<DV>;
  constexpr int NCQ = (TQ::CHUNKS + 255) / 256, NCV = (TV::CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][TQ::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Os[2][TV::ELEMS];  // dO tiles
  __shared__ float St[2][2][BT];                                  // lse, delta of the tile's queries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int S = a.S, nb = (S + BROWS - 1) / BROWS;
  int bh, blk;
  block_of(a.BH, nb, bh, blk, false);  // early key blocks see the most queries
  const int64_t hoff = (int64_t)bh * S;
  const bf16 *q = reinterpret_cast<const bf16 *>(a.q) + hoff * DQK;
  const bf16 *k = reinterpret_cast<const bf16 *>(a.k) + hoff * DQK;
  const bf16 *v = reinterpret_cast<const bf16 *>(a.v) + hoff * DV;
  const bf16 *dout = reinterpret_cast<const bf16 *>(a.dout) + hoff * DV;
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
  uint4 rq[NCQ], ro[NCV];
  float rst = 0.f;
  auto load = [&](int t) {
    load_tile<DQK, NCQ>(q, t * BT, S, tid, rq);
    load_tile<DV, NCV>(dout, t * BT, S, tid, ro);
    if (tid < 2 * BT) {
      const int qq = t * BT + (tid & (BT - 1));
      rst = qq < S ? (tid < BT ? a.lse : a.delta)[hoff + qq] : 0.f;
    }
  };
  auto store = [&](int buf) {
    store_tile<DQK, NCQ>(Qs[buf], tid, rq);
    store_tile<DV, NCV>(Os[buf], tid, ro);
    if (tid < 2 * BT) St[buf][tid / BT][tid & (BT - 1)] = rst;
  };
  load(t0);
  store(0);
  __syncthreads();
  for (int t = t0; t < ntiles; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < ntiles) load(t + 1);
    // queries of tile t that this wave's keys can see: qi >= kj for some lane
    if (t * BT + BT - 1 >= kw) {
      const bf16 *qt = Qs[buf], *ot = Os[buf];
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<TQ::PITCH>(qt, l32, g, f), kf[f], s, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NVF; ++f)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<TV::PITCH>(ot, l32, g, f), vf[f], dp, 0, 0, 0);
      // P and dS: row r is query t BT + acc_row(r), the lane's column key kj
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = acc_row(r, lane), qi = t * BT + qr;
        const float p = (kj <= qi && qi < S) ? __builtin_amdgcn_exp2f(s[r] * sl2 - St[buf][0][qr]) : 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - St[buf][1][qr]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pa = pack8(s, u), da = pack8(dp, u);
#pragma unroll
        for (int d = 0; d < NVT; ++d)
          dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, col_frag<TV::PITCH>(ot, lane, u, d), dv[d], 0, 0, 0);
#pragma unroll
        for (int d = 0; d < NKT; ++d)
          dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, col_frag<TQ::PITCH>(qt, lane, u, d), dk[d], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) store(buf ^ 1);
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
  using TK = TileLds<DQK>;
  using TV = TileLds<DV>;
  constexpr int NCK = (TK::CHUNKS + 255) / 256, NCV = (TV::CHUNKS + 255) / 256;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TK::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][TV::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
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
  const float lse = qi < S ? a.lse[hoff + qi] : 0.f, delta = qi < S ? a.delta[hoff + qi] : 0.f;
  f32x16 dq[NKT];
#pragma unroll
  for (int d = 0; d < NKT; ++d) dq[d] = f32x16{};
  const float sl2 = a.scale * BLOG2E;
  const int ntiles = (min(S, q0 + BROWS) + BT - 1) / BT;
  const int last = (qw + BT - 1) / BT;
  uint4 rk[NCK], rv[NCV];
  load_tile<DQK, NCK>(k, 0, S, tid, rk);
  load_tile<DV, NCV>(v, 0, S, tid, rv);
  store_tile<DQK, NCK>(Ks[0], tid, rk);
  store_tile<DV, NCV>(Vs[0], tid, rv);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      load_tile<DQK, NCK>(k, (t + 1) * BT, S, tid, rk);
      load_tile<DV, NCV>(v, (t + 1) * BT, S, tid, rv);
    }
    if (t <= last) {
      const bf16 *kt = Ks[buf], *vt = Vs[buf];
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int f = 0; f < NQF; ++f)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<TK::PITCH>(kt, l32, g, f), qf[f], s, 0, 0, 0);
#pragma unroll
      for (int f = 0; f < NVF; ++f)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<TV::PITCH>(vt, l32, g, f), of[f], dp, 0, 0, 0);
      // row r is key t BT + acc_row(r), the lane's column query qi
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = t * BT + acc_row(r, lane);
        const float p = (kj <= qi && qi < S) ? __builtin_amdgcn_exp2f(s[r] * sl2 - lse) : 0.f;
        dp[r] = p * (dp[r] - delta);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 da = pack8(dp, u);
#pragma unroll
        for (int d = 0; d < NKT; ++d)
          dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, col_frag<TK::PITCH>(kt, lane, u, d), dq[d], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) {
      store_tile<DQK, NCK>(Ks[buf ^ 1], tid, rk);
      store_tile<DV, NCV>(Vs[buf ^ 1], tid, rv);
    }
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
