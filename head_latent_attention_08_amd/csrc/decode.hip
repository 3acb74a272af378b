// Absorbed MLA decode attention over the latent cache (gfx950).
//
// The cache formula of "The Evolving Transformer -- DeepSeek V2 & V3" (section
// 01: c_kv is cached; K_i and V_i are per-head up-projections of c_kv) lets the
// per-head up-projections move onto the query and output sides:
//   s_h,t = scale (q_lat_h . c_kv_t + q_pe_h . k_pe_t),  q_lat_h = W_uk_h^T q_nope_h
//   o_lat_h = sum_t softmax_t(s_h) c_kv_t,               o_h = W_uv_h o_lat_h
// so every head reads the same 576-wide cache rows [c_kv ‖ k_pe].  This kernel
// streams each row from HBM once for all heads of a head group.
//
// Work split: the rows of all sequences (lens[b] + q_len each, the new
// tokens included) are laid end to end, each non-empty sequence preceded by
// PIECE_COST_ROWS virtual rows standing for the cost of starting a piece,
// and cut into n_blocks equal ranges, so long and short sequences load the
// GPU evenly.  Each range is processed by one workgroup per group of 128
// query heads (a single one at 128 heads and one token, so every cache row
// leaves HBM once); with more head groups the workgroups of a range are
// numbered so they land on the same XCD (workgroup ids go to the eight XCDs
// round-robin) and the repeated reads of a cache tile hit that XCD's L2.  A
// range that spans sequence boundaries yields one partial (unnormalised
// o_lat, running max, running sum) per sequence piece, in slot (range + b)
// -- unique because range and sequence indices both rise along the rows.  A
// merge kernel combines the pieces of each sequence with log-sum-exp weights.
// With a bf16 cache the partial o_lat is stored in bf16 (half the bytes the
// attention kernel writes and the merge reads back, one extra rounding that
// the final bf16 output would mostly absorb); with fp32 it stays fp32.
//
// Inside a workgroup: four waves, 32 heads each (one head per lane pair), on
// 32x32x16 MFMAs.  A wave computes S^T = C Q^T (32 cache rows x 32 heads per
// tile, K = 576), keeps the softmax online per head, and accumulates
// O^T += C^T P^T with P^T taken from the score accumulators in place.  The
// C^T operand comes straight from the row-major cache tile through the 16-bit
// transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes 4e + i / 4 (e = 0..3), so
// pointing lane s at row j0 + s / 4, column c0 + 4 (s % 4) hands every lane
// keys j0..j0+3 of its own column c0 + i.  Cache tiles of 32 rows stream
// from HBM straight into three LDS stages (global_load_lds, 16 bytes a lane,
// issued two tiles ahead), so no staging registers are needed.  The
// softmax reference max of a sequence piece is the max of its first tile and
// is never moved, so the 256 accumulators per lane are never rescaled (a
// rescale would pull them through the vector registers); a score more than
// 2^64 above the reference makes the piece run again with its true max.
// Thirty-two heads per wave keep LDS reads at four per tile per workgroup;
// to leave room for the 256 accumulators, the last query channels are read
// from LDS each tile instead of being held in registers.

#include "common.h"
#include "internal.h"

#include <type_traits>

namespace mla {
namespace {

constexpr int TK = 32;    // cache rows per tile
constexpr int HPW = 32;   // heads per wave
constexpr int HPB = 128;  // heads per workgroup
constexpr int DTHREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
// a segment's reference max is its first tile's max; scores may exceed it
// by up to 2^64 (exp2 domain) before fp32 sums could overflow
constexpr float HEADROOM_LOG2 = 64.0f;

template <typename T, int R, int DR>
struct DecCfg {
  using MF = Mfma32<T>;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int W = R + DR;
  static constexpr int WP = (W + MF::KSTEP - 1) / MF::KSTEP * MF::KSTEP;
  static constexpr int RP = (R + 31) / 32 * 32;
  // Rows whose width is a whole number of 128-byte groups (bf16 at V3
  // sizes: 1152 B) are stored unpadded with their 16-byte chunks permuted
  // within each group of eight (dec_swz), which keeps both the row-wise
  // 16-byte reads of the score step and the transposing 8-byte reads of the
  // output step free of bank conflicts, and makes a stage an exact number of
  // copy instructions.  Other shapes use a padded pitch.
  static constexpr bool SWZ = sizeof(T) == 2 && (W * 2) % 128 == 0 && WP == W && RP <= W;
  static constexpr int CPITCH = SWZ ? W : (WP > RP ? WP : RP) + VEC;
  static constexpr int ROWB = CPITCH * (int)sizeof(T);       // row pitch in bytes
  // a stage is whole 1 KB blocks: one DMA instruction fills 64 lanes x 16 B
  static constexpr int NINS = (TK * ROWB + 1023) / 1024;
  static constexpr int STAGEB = NINS * 1024;
  static constexpr int NQF = WP / MF::KSTEP;
  // the first NQR query fragments live in registers, the rest in LDS
  static constexpr int NQR = NQF > 26 ? 26 : NQF;
  static constexpr int NQL = NQF - NQR;
  static constexpr int QPITCH = NQL * MF::KSTEP + VEC;
  static constexpr int NCT = RP / 32;
};

// Four consecutive channels of a split partial as stored: bf16 for a bf16
// cache (the only 2-byte element type here), else fp32.
template <typename T> struct Part4 {
  static constexpr bool NARROW = sizeof(T) == 2;
  using elem = std::conditional_t<NARROW, T, float>;
  using raw = std::conditional_t<NARROW, uint2, f32x4>;
  __device__ static raw pack(float a, float b, float c, float d) {
    if constexpr (NARROW) {
      const bf16x2 lo = {from_f32<T>(a), from_f32<T>(b)};
      const bf16x2 hi = {from_f32<T>(c), from_f32<T>(d)};
      return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    } else {
      return f32x4{a, b, c, d};
    }
  }
  __device__ static f32x4 unpack(raw r) {
    if constexpr (NARROW) {  // a bf16 is the upper half of the fp32 with its bits
      return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                   __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    } else {
      return r;
    }
  }
};

constexpr int NSTAGE = 3;  // cache tiles in flight: current, next, and the one after

// Chunk permutation of the swizzled stage layout: in row r, logical 16-byte
// chunk c sits at position (c & ~7) | ((c & 7) ^ dec_swz(r)).  Rows 2m and
// 2m+1 share a value and fall 32 banks apart; the values of the eight pairs
// in 16 rows are distinct, and rows 4i, 4i+2 differ in bit 2.
__device__ inline int dec_swz(int row) {
  const int m = (row >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; expcnt and lgkmcnt left open).
#define DEC_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Rows of sequence b: lens[b] + q_len (the cached prefix and the new
// tokens) for a valid length, else 0.
__device__ inline int seq_rows(const int32_t *lens, int b, int64_t cap, int q_len) {
  const int32_t L = lens[b];
  return (L >= 0 && (int64_t)L + q_len <= cap) ? L + q_len : 0;
}

// Starting a sequence piece (query loads, first tiles in flight, partial
// stores) costs a workgroup about as much as this many rows of the tile
// loop.  The rows are laid end to end with this many virtual rows in front
// of every non-empty sequence before the total is cut into equal ranges, so
// a range that starts a second sequence gets that many fewer real rows.
constexpr int PIECE_COST_ROWS = 384;
__device__ inline int seq_vrows(const int32_t *lens, int b, int64_t cap, int q_len) {
  const int n = seq_rows(lens, b, cap, q_len);
  return n > 0 ? n + PIECE_COST_ROWS : 0;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T, int R, int DR>
__global__ __launch_bounds__(DTHREADS) void decode_attn_kernel(DecodeAttnArgs a) {
  using C = DecCfg<T, R, DR>;
  using MF = typename C::MF;
  constexpr int VEC = C::VEC, W = C::W, CPITCH = C::CPITCH, ROWB = C::ROWB, NINS = C::NINS,
                STAGEB = C::STAGEB, NQF = C::NQF, NQR = C::NQR, NQL = C::NQL, QPITCH = C::QPITCH,
                NCT = C::NCT;
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGEB];
  __shared__ __attribute__((aligned(16))) T Qs[NQL > 0 ? HPB * QPITCH : VEC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int g = lane >> 5, l32 = lane & 31;
  const int B = a.B, H = a.H;
  const int n_hg = (H + HPB - 1) / HPB;
  // workgroup -> (range, head group); head groups of one range share an XCD
  int blk, hg;
  if ((a.n_blocks & 7) == 0) {
    const int local = blockIdx.x >> 3;
    hg = local % n_hg;
    blk = (local / n_hg) * 8 + (blockIdx.x & 7);
  } else {
    hg = blockIdx.x % n_hg;
    blk = blockIdx.x / n_hg;
  }
  const int h = hg * HPB + wave * HPW + l32;
  const bool wave_live = hg * HPB + wave * HPW < H;

  // The virtual rows (seq_vrows) of the sequences laid end to end: the
  // total, cut into n_blocks equal ranges, and the first sequence holding
  // row r0 with the row it starts at.  Every wave works these out by itself
  // (64 sequences per step, an in-register prefix sum), so no LDS and no
  // barrier depend on the batch size.
  int total = 0;
  for (int b0 = lane; b0 < B; b0 += 64) total += seq_vrows(a.lens, b0, a.cap, a.q_len);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o);
  total = __builtin_amdgcn_readfirstlane(total);  // the same in every lane
  const int per = (total + a.n_blocks - 1) / a.n_blocks;
  int r0 = blk * per;
  const int r1 = min(r0 + per, total);
  if (r0 >= r1) return;
  int b = 0, sb = 0;  // sequence b starts at virtual row sb
  for (int c0 = 0; c0 < B; c0 += 64) {
    const int i = c0 + lane;
    int v = i < B ? seq_vrows(a.lens, i, a.cap, a.q_len) : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    const int ends = sb + v;  // end of sequence i
    const int n = __popcll(__ballot(i < B && ends <= r0));
    b = c0 + n;
    if (n < 64) {
      if (n > 0) sb = __builtin_amdgcn_readlane(ends, n - 1);
      break;
    }
    sb = __builtin_amdgcn_readlane(ends, 63);
  }

  const float sl2 = a.scale * LOG2E;
  const char *cache = reinterpret_cast<const char *>(a.cache);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)lds;
  // DMA instructions per tile issued by this wave (instructions wave, wave+4, ..)
  const int n_dma = (NINS - wave + 3) / 4;
  // this lane's byte offset from a tile's first row and its row, per copy
  // instruction (padding and out-of-tile lanes: offset 0, row 0)
  constexpr int NPW = (NINS + 3) / 4;
  uint32_t dof[NPW];
  int drow[NPW];
#pragma unroll
  for (int k = 0; k < NPW; ++k) {
    const int o = (wave + 4 * k) * 1024 + lane * 16;
    const int row = o / ROWB, cbyte = o - row * ROWB;
    const bool ok = wave + 4 * k < NINS && row < TK && cbyte < W * (int)sizeof(T);
    int src = cbyte;  // byte of the cache row this lane's 16 bytes come from
    if constexpr (C::SWZ) {
      const int pch = cbyte >> 4;
      src = ((pch & ~7) | ((pch & 7) ^ dec_swz(row))) << 4;
    }
    dof[k] = ok ? (uint32_t)(row * W * (int)sizeof(T) + src) : 0u;
    drow[k] = ok ? row : 0;
  }

  // swizzled layout: element offset of this lane's score-step chunk
  // 2 f + g of row l32 is kofs[f % 4] + 64 (f / 4)
  int kofs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kofs[i] = l32 * CPITCH + (((2 * i + g) ^ dec_swz(l32)) << 3);

  // this lane's new token: query head h is token h / heads_per_tok's head
  const int hpt = a.heads_per_tok > 0 ? a.heads_per_tok : H;
  const int tok = min(h, H - 1) / hpt;

  while (r0 < r1 && b < B) {
    // sequence b's real rows sit at [rs, re) of the virtual row axis
    const int re = sb + seq_vrows(a.lens, b, a.cap, a.q_len);
    const int rs = re > sb ? sb + PIECE_COST_ROWS : re;
    const int pb = max(r0, rs), pe = min(r1, re);
    if (pb >= pe) {  // only virtual rows of b in this range (uniform)
      r0 = re;
      sb = re;
      ++b;
      continue;
    }
    const int t_begin = pb - rs, t_end = pe - rs;
    // token tok sees rows 0 .. lens[b] + tok, i.e. all but the last
    // q_len - 1 - tok rows of the sequence; t_end_min is the lowest such
    // limit among the lanes (all of them at q_len = 1)
    const int rows_b = re - rs;
    const int t_lim = min(t_end, rows_b - (a.q_len - 1 - tok));
    const int t_end_min = min(t_end, rows_b - (a.q_len - 1));
    const char *cb = cache + (int64_t)b * a.cap * W * (int64_t)sizeof(T);

    // Cache tile t0 -> stage: instruction i of the stage fills bytes
    // [1024 i, 1024 i + 1024) of the stage, lane l the 16 bytes at 16 l.  A
    // lane whose bytes fall on the row padding or past the segment copies
    // the tile's first chunk instead (finite data that is never read as a
    // valid row: those rows are masked, the padding columns meet zero
    // queries or output channels >= R).  The lane's offset from the tile's
    // first row is fixed (dof, drow); the tile base is a scalar.
    // Written as inline asm with explicit vmcnt waits: the compiler builtin for
    // this load makes every later LDS read wait for all outstanding copies,
    // which would serialise the two-tiles-ahead pipeline.
#define DEC_ROW0(T0)                                                                     \
  [&] {                                                                                  \
    const uint64_t r0a_ = (uint64_t)(cb + (int64_t)(T0) * W * (int64_t)sizeof(T));       \
    return reinterpret_cast<const char *>(                                               \
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(r0a_ >> 32)) << 32) |       \
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r0a_));             \
  }()
    // copy instruction k of this wave for the tile whose first row is ROW0
    // (LIM rows of it valid) into stage STG
#define DEC_DMA_INS(STG, ROW0, LIM, K)                                                   \
  do {                                                                                   \
    const int ins_ = wave + 4 * (K);                                                     \
    if ((K) < NPW && ins_ < NINS) {                                                      \
      const uint32_t off_ = drow[(K) < NPW ? (K) : 0] < (LIM) ? dof[(K) < NPW ? (K) : 0] : 0u; \
      const uint32_t m0 = lds_base + (STG) * STAGEB + ins_ * 1024;                       \
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"                    \
                   :                                                                     \
                   : "v"(off_), "s"(ROW0), "s"(m0)                                       \
                   : "memory", "m0");                                                    \
    }                                                                                    \
  } while (0)
#define DEC_DMA(STG, T0)                                                                 \
  do {                                                                                   \
    const char *row0_ = DEC_ROW0(T0);                                                    \
    const int lim_ = t_end - (T0);                                                       \
    _Pragma("unroll") for (int k = 0; k < NPW; ++k) DEC_DMA_INS(STG, row0_, lim_, k);    \
  } while (0)

    const int ntiles = (t_end - t_begin + TK - 1) / TK;
    // Query fragments first (the loads of all workgroups at once are the
    // start-up burst; copies issued before them would stall the wave at
    // issue).  Then every wave has left the previous piece's tile loop, so
    // its stages and query rows are free for the query rows and the first
    // two tiles.
    // B operand of S^T = C Q^T: lane holds head l32, k values g*KPL.. of a step
    typename MF::frag qf[NQR];
    const T *qp = reinterpret_cast<const T *>(a.q_lat) + ((int64_t)b * H + h) * W;
#pragma unroll
    for (int f = 0; f < NQR; ++f) {
      const int c = f * MF::KSTEP + g * MF::KPL;
      if constexpr (MF::KPL == 1) {
        qf[f] = (h < H && c < W) ? to_f32(qp[c]) : 0.f;
      } else {
        if (h < H && c < W) {
          uint4 v = *reinterpret_cast<const uint4 *>(qp + c);
          qf[f] = *reinterpret_cast<typename MF::frag *>(&v);
        } else {
#pragma unroll
          for (int e = 0; e < MF::KPL; ++e) qf[f][e] = from_f32<T>(0.f);
        }
      }
    }
    __syncthreads();
    if constexpr (NQL > 0) {
      // query channels NQR*KSTEP.. of this workgroup's heads; the first
      // tile's barrier publishes them
      constexpr int QCH = NQL * MF::KSTEP / VEC;
      for (int i = tid; i < HPB * QCH; i += DTHREADS) {
        const int hh = i / QCH, cc = (i - hh * QCH) * VEC;
        const int hq = hg * HPB + hh;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (hq < H && NQR * MF::KSTEP + cc < W)
          v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const T *>(a.q_lat) +
                                               ((int64_t)b * H + hq) * W + NQR * MF::KSTEP + cc);
        *reinterpret_cast<uint4 *>(&Qs[hh * QPITCH + cc]) = v;
      }
    }
    if (ntiles > 0) DEC_DMA(0, t_begin);
    if (ntiles > 1) DEC_DMA(1, t_begin + TK);
    f32x16 o[NCT];
    float m_ref = -INFINITY, m_true = -INFINITY, l_run = 0.f;
    bool ovf = false;
    // The softmax reference max is fixed at the first tile, so the
    // accumulators are never rescaled inside the loop (they stay in the MFMA
    // accumulation registers).  A score more than 2^64 above it sets ovf and
    // the segment is run a second time with the true max, known by then.
    for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      // every wave is past its tile loop here, so the stages are free
      if (!__syncthreads_or(ovf)) break;
      m_ref = m_true;
      ovf = false;
      DEC_DMA(0, t_begin);
      if (ntiles > 1) DEC_DMA(1, t_begin + TK);
    }
#pragma unroll
    for (int d = 0; d < NCT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    l_run = 0.f;
    int rd = 0;
    for (int it = 0; it < ntiles; ++it) {
      const int t0 = t_begin + it * TK;
      // this wave's copies of tile it are in LDS once at most the next tile's
      // instructions are outstanding; the barrier publishes every wave's copy
      // and frees the stage read in the previous iteration
      if (it + 1 < ntiles) {
        if (n_dma == NINS / 4) __builtin_amdgcn_s_waitcnt(DEC_VMCNT(NINS / 4));
        else __builtin_amdgcn_s_waitcnt(DEC_VMCNT((NINS + 3) / 4));
      } else {
        __builtin_amdgcn_s_waitcnt(DEC_VMCNT(0));
      }
      __syncthreads();
      // stage rd holds tile it; tile it + 2 goes to the stage read last time.
      // A live wave spreads its copy instructions over the score MFMAs (issued
      // in a burst, the copies of all four waves queue behind each other).
      const bool dma_next = it + 2 < ntiles;
      const int dstg = rd == 0 ? NSTAGE - 1 : rd - 1;
      const char *drow0 = DEC_ROW0(t0 + 2 * TK);
      const int dlim = t_end - (t0 + 2 * TK);
      if (!wave_live && dma_next) {
#pragma unroll
        for (int k = 0; k < NPW; ++k) DEC_DMA_INS(dstg, drow0, dlim, k);
      }
      const T *cs = reinterpret_cast<const T *>(lds + __builtin_amdgcn_readfirstlane(rd * STAGEB));
      rd = rd == NSTAGE - 1 ? 0 : rd + 1;
      if (wave_live) {
        // S^T = C Q^T; fragment reads run two MFMAs ahead (the fences keep
        // the compiler from hoisting all of them)
        f32x16 st;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = 0.f;
        typename MF::frag ka[2], qa[2], kb[2], qb[2];
#define DEC_KLOAD(KA, QA, F0)                                                         \
  _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                     \
    const int f_ = (F0) + e;                                                          \
    if (f_ < NQF) {                                                                   \
      const int c_ = f_ * MF::KSTEP + g * MF::KPL;                                    \
      if constexpr (MF::KPL == 1) {                                                   \
        KA[e] = to_f32(cs[l32 * CPITCH + c_]);                                        \
        if (f_ >= NQR) QA[e] = to_f32(Qs[(wave * HPW + l32) * QPITCH + c_ - NQR * MF::KSTEP]); \
      } else {                                                                        \
        KA[e] = *reinterpret_cast<const typename MF::frag *>(                          \
            &cs[C::SWZ ? kofs[f_ & 3] + 64 * (f_ >> 2) : l32 * CPITCH + c_]);           \
        if (f_ >= NQR)                                                                \
          QA[e] = *reinterpret_cast<const typename MF::frag *>(                       \
              &Qs[(wave * HPW + l32) * QPITCH + c_ - NQR * MF::KSTEP]);               \
      }                                                                               \
    }                                                                                 \
  }
#define DEC_KMMA(KA, QA, F0)                                                          \
  _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                     \
    const int f_ = (F0) + e;                                                          \
    if (f_ < NQF) st = MF::mma(KA[e], f_ < NQR ? qf[f_ < NQR ? f_ : 0] : QA[e], st);  \
  }
        DEC_KLOAD(ka, qa, 0)
        constexpr int NIT = (NQF + 3) / 4;  // score steps of four MFMAs
#pragma unroll
        for (int f0 = 0; f0 < NQF; f0 += 4) {
          if (dma_next) {
            // copy instructions [j NPW / NIT, (j + 1) NPW / NIT) at step j
#pragma unroll
            for (int k = f0 / 4 * NPW / NIT; k < (f0 / 4 + 1) * NPW / NIT; ++k)
              DEC_DMA_INS(dstg, drow0, dlim, k);
          }
          DEC_KLOAD(kb, qb, f0 + 2)
          __builtin_amdgcn_sched_barrier(0);
          DEC_KMMA(ka, qa, f0)
          __builtin_amdgcn_sched_barrier(0);
          DEC_KLOAD(ka, qa, f0 + 4)
          __builtin_amdgcn_sched_barrier(0);
          DEC_KMMA(kb, qb, f0 + 2)
          __builtin_amdgcn_sched_barrier(0);
        }
#undef DEC_KLOAD
#undef DEC_KMMA
        if (t0 + TK > t_end_min) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + acc_row(r, lane) >= t_lim) st[r] = -INFINITY;
        }
        float mx = st[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        m_true = fmaxf(m_true, mx);
        if (m_ref == -INFINITY) m_ref = mx;  // first tile of the segment
        if ((mx - m_ref) * sl2 > HEADROOM_LOG2) ovf = true;
        // a lane whose rows of this piece are all past its token's limit
        // keeps m_ref = -inf: its probabilities are exp2(-inf) = 0
        const float neg = m_ref == -INFINITY ? 0.f : -m_ref * sl2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st[r] = __builtin_amdgcn_exp2f(fmaf(st[r], sl2, neg));
          l_run += st[r];
        }
        // O^T += C^T P^T
        if constexpr (MF::KPL == 1) {
#pragma unroll
          for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int d = 0; d < NCT; ++d)
              o[d] = MF::mma(to_f32(cs[acc_row(t, lane) * CPITCH + d * 32 + l32]), st[t], o[d]);
        } else {
          // k slots e of MFMA u: keys 16u + (e/4)*8 + 4g + e%4, matching the
          // score accumulator layout
          const int s16 = lane & 15;
          const T *pb0 = &cs[(4 * g + (s16 >> 2)) * CPITCH + (lane & 16) + 4 * (s16 & 3)];
          // swizzled layout: rows 16u + 4g + s16/4 (+ 8 for the upper four
          // keys), chunk 4D + x, x = (lane & 16)/8 + (s16 & 3)/2; the permuted
          // position is 4 (D ^ fb) + (x ^ (f & 3)), fb = f / 4, so the offset
          // is a per-lane base +- 32 fb for even / odd D plus 32 D
          int vofs[2][2][2];  // [u][upper][D odd]
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
              const int rr = 16 * u + 4 * g + (s16 >> 2) + 8 * hi;
              const int fr = dec_swz(rr);
              const int x = ((lane & 16) >> 3) + ((s16 & 3) >> 1);
              const int base = rr * CPITCH + ((x ^ (fr & 3)) << 3) + 4 * (s16 & 1);
              const int fb = fr >> 2;
              vofs[u][hi][0] = base + 32 * fb;
              vofs[u][hi][1] = base - 32 * fb;
            }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            typename MF::frag pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = from_f32<T>(st[u * 8 + e]);
            typename MF::frag vf[NCT];
#define DEC_VLOAD(D)                                                                    \
  if ((D) < NCT) {                                                                      \
    const T *p_ = C::SWZ ? cs + vofs[u][0][(D) & 1] + (D) * 32 : pb0 + u * 16 * CPITCH + (D) * 32; \
    const T *q_ = C::SWZ ? cs + vofs[u][1][(D) & 1] + (D) * 32 : p_ + 8 * CPITCH;      \
    const s16x4 lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                          \
        (__attribute__((address_space(3))) s16x4 *)(p_));                               \
    const s16x4 hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                          \
        (__attribute__((address_space(3))) s16x4 *)(q_));                               \
    vf[(D) < NCT ? (D) : 0] =                                                           \
        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7)); \
  }
            DEC_VLOAD(0)
            DEC_VLOAD(1)
#pragma unroll
            for (int d = 0; d < NCT; ++d) {
              DEC_VLOAD(d + 2)
              __builtin_amdgcn_sched_barrier(0);
              o[d] = MF::mma(vf[d], pf, o[d]);
              __builtin_amdgcn_sched_barrier(0);
            }
#undef DEC_VLOAD
          }
        }
      }
    }
    }  // pass

    // partial of this sequence piece: unnormalised o_lat (log2-domain max,
    // sum).  o_lat is stored in the accumulator layout, 32 heads x RP
    // channels per block: channel tile d, row quad q, lane, 4 values, so each
    // store instruction writes consecutive bytes (1 KB in fp32, 512 B in bf16).
    using P4 = Part4<T>;
    typename P4::elem *po =
        reinterpret_cast<typename P4::elem *>(a.part_o) +
        ((int64_t)(blk + b) * ((H + HPW - 1) / HPW) + hg * (HPB / HPW) + wave) * (HPW * NCT * 32) + lane * 4;
    // channel tiles per wave per round of the LDS bounce below
    constexpr int DPR = NSTAGE * STAGEB / (4 * 4 * 1024) < NCT ? NSTAGE * STAGEB / (4 * 4 * 1024) : NCT;
    if constexpr (P4::NARROW && DPR >= 1) {
      // The accumulators pass through the idle cache stages: each lane
      // writes its fp32 quads to LDS and reads them back into vector
      // registers to convert them.  Converting straight from the
      // accumulation registers moves the MFMAs' accumulators to the vector
      // registers, where they do not fit beside the tile loop's operands.
      // Every wave is past its tile loop once the first barrier is passed;
      // a lane reads only what it wrote, and the barriers keep the stores
      // and loads in order.  (Shapes whose stages are too small for this
      // have few accumulators and convert them directly.)
      f32x4 *bounce = reinterpret_cast<f32x4 *>(lds + wave * (DPR * 4 * 1024)) + lane;
#pragma unroll
      for (int d0 = 0; d0 < NCT; d0 += DPR) {
        __syncthreads();
        if (wave_live) {
#pragma unroll
          for (int dd = 0; dd < DPR; ++dd)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (d0 + dd < NCT)
                bounce[(dd * 4 + q) * 64] = f32x4{o[d0 + dd][4 * q], o[d0 + dd][4 * q + 1],
                                                  o[d0 + dd][4 * q + 2], o[d0 + dd][4 * q + 3]};
        }
        __syncthreads();
        if (wave_live) {
#pragma unroll
          for (int dd = 0; dd < DPR; ++dd)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (d0 + dd < NCT) {
                const f32x4 v = bounce[(dd * 4 + q) * 64];
                *reinterpret_cast<typename P4::raw *>(po + ((d0 + dd) * 4 + q) * 256) =
                    P4::pack(v[0], v[1], v[2], v[3]);
              }
        }
      }
    } else if (wave_live) {
#pragma unroll
      for (int d = 0; d < NCT; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<typename P4::raw *>(po + (d * 4 + q) * 256) =
              P4::pack(o[d][4 * q], o[d][4 * q + 1], o[d][4 * q + 2], o[d][4 * q + 3]);
    }
    if (wave_live) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const int slot = blk + b;
      if (h < H && g == 0) {
        a.part_ml[((int64_t)slot * H + h) * 2 + 0] = m_ref * sl2;
        a.part_ml[((int64_t)slot * H + h) * 2 + 1] = l_tot;
      }
    }
    r0 = re;
    sb = re;
    ++b;
  }
#undef DEC_DMA
#undef DEC_DMA_INS
#undef DEC_ROW0
}

// Combine the pieces of sequence b: o_lat = sum_i w_i O_i / sum_i w_i l_i,
// w_i = exp2(m_i - max_i m_i).  A sequence with no valid rows gets NaN.
// One workgroup per (sequence, block of 32 heads).  A piece's block is 32
// heads x RP channels in the attention kernel's accumulator layout (16-byte
// chunk k holds lane k % 64 of accumulator quad k / 64: head k % 32,
// channels (k / 256) * 32 + (k / 64 % 4) * 8 + (k % 64 / 32) * 4 + 0..3), so
// thread t reads chunks t, t + 256, .. -- whole 1 KB runs per wave -- and
// they all belong to one head.
constexpr int MERGE_MAXP = 264;  // pieces per sequence: at most n_blocks + 1

template <typename T, int R>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  constexpr int RP = (R + 31) / 32 * 32;
  constexpr int NCH = HPW * RP / 4 / 256;  // chunks per thread (RP / 32)
  __shared__ int sh[2];
  __shared__ float wsh[HPW][MERGE_MAXP], lsh[HPW][MERGE_MAXP];
  const int b = blockIdx.x, hb = blockIdx.y, tid = threadIdx.x;
  if (tid < 64) {
    int before = 0, all = 0;
    for (int i = tid; i < a.B; i += 64) {
      const int n = seq_vrows(a.lens, i, a.cap, a.q_len);
      all += n;
      if (i < b) before += n;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      before += __shfl_xor(before, o);
      all += __shfl_xor(all, o);
    }
    if (tid == 0) {
      sh[0] = before;
      sh[1] = all;
    }
  }
  __syncthreads();
  const int start = sh[0], total = sh[1];
  const int n_b = seq_rows(a.lens, b, a.cap, a.q_len);
  const int lane = tid & 63, hl = lane & 31, g = lane >> 5;
  const int h = hb * HPW + hl;
  T *out = reinterpret_cast<T *>(a.o_lat) + ((int64_t)b * a.H + h) * R;
  if (n_b == 0) {
    if (h < a.H)
      for (int k = 0; k < NCH; ++k) {
        const int c = (k * 4 + (tid >> 6)) * 8 + g * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < R) out[c + e] = from_f32<T>(NAN);
      }
    return;
  }
  // pieces: the ranges that hold the real rows [start + PIECE_COST_ROWS, + n_b)
  // of the virtual row axis
  const int per = (total + a.n_blocks - 1) / a.n_blocks;
  const int i0 = (start + PIECE_COST_ROWS) / per, i1 = (start + PIECE_COST_ROWS + n_b - 1) / per;
  const int np = i1 - i0 + 1;  // <= n_blocks + 1 <= MERGE_MAXP (checked on the host)
  // piece weights w_i / L of the block's heads: the (max, sum) pairs of all
  // pieces are loaded in parallel into LDS, then one thread per head reduces
  for (int idx = tid; idx < HPW * np; idx += 256) {
    const int hw = idx % HPW, i = idx / HPW;
    float2 ml = make_float2(-INFINITY, 0.f);
    if (hb * HPW + hw < a.H)
      ml = *reinterpret_cast<const float2 *>(a.part_ml + ((int64_t)(i0 + i + b) * a.H + hb * HPW + hw) * 2);
    wsh[hw][i] = ml.x;
    lsh[hw][i] = ml.y;
  }
  __syncthreads();
  if (tid < HPW) {
    float M = -INFINITY;
    for (int i = 0; i < np; ++i) M = fmaxf(M, wsh[tid][i]);
    float L = 0.f;
    for (int i = 0; i < np; ++i) L += exp2f(wsh[tid][i] - M) * lsh[tid][i];
    const float invL = 1.0f / L;
    for (int i = 0; i < np; ++i) wsh[tid][i] = exp2f(wsh[tid][i] - M) * invL;
  }
  __syncthreads();
  const int n_hb = (a.H + HPW - 1) / HPW;
  f32x4 acc[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (h < a.H) {
    // two register sets: the loads of piece i + 1 are in flight while piece
    // i is accumulated (loads past the last piece re-read it and are not
    // used; unconditional loads keep the wait counts exact)
    using P4 = Part4<T>;
    using raw = typename P4::raw;
    const raw *po = reinterpret_cast<const raw *>(reinterpret_cast<const typename P4::elem *>(a.part_o) +
                                                  ((int64_t)(i0 + b) * n_hb + hb) * (HPW * RP)) +
                    tid;
    const int64_t pstride = (int64_t)n_hb * HPW * RP / 4;  // four-channel chunks per piece
    raw va[NCH], vb[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) va[k] = po[k * 256];
    for (int i = 0; i < np; i += 2) {
      const raw *pb = po + min(i + 1, np - 1) * pstride;
#pragma unroll
      for (int k = 0; k < NCH; ++k) vb[k] = pb[k * 256];
      const float wa = wsh[hl][i];
      const float wb = i + 1 < np ? wsh[hl][i + 1] : 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k) acc[k] += wa * P4::unpack(va[k]);
      const raw *pa = po + min(i + 2, np - 1) * pstride;
#pragma unroll
      for (int k = 0; k < NCH; ++k) va[k] = pa[k * 256];
#pragma unroll
      for (int k = 0; k < NCH; ++k) acc[k] += wb * P4::unpack(vb[k]);
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = (k * 4 + (tid >> 6)) * 8 + g * 4;
      if constexpr (sizeof(T) == 2 && R % 4 == 0) {
        if (c < R) {
          const bf16x2 lo = {from_f32<T>(acc[k][0]), from_f32<T>(acc[k][1])};
          const bf16x2 hi = {from_f32<T>(acc[k][2]), from_f32<T>(acc[k][3])};
          *reinterpret_cast<uint2 *>(out + c) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < R) out[c + e] = from_f32<T>(acc[k][e]);
      }
    }
  }
}

// Absorption q_lat[b, h, :] = W_uk_h^T q_nope[b, h] (bf16): one workgroup per
// (head, 128 latent channels, 64 sequences).  The head's W_uk rows (k = nope
// channel, n = latent channel, n contiguous) are staged in LDS; the MFMA B
// operand needs 8 consecutive k of one n per lane, read with the 16-bit
// transposing LDS read (lane s of a 16-lane group addresses row k0 + s/4,
// columns n0 + 4 (s%4) .. +3; lane i then holds rows k0..k0+3 of column
// n0 + i).  q_nope rows are the A operand straight from global memory.
constexpr int AB_N = 128, AB_M = 64;

template <int DN>
__global__ __launch_bounds__(256) void absorb_kernel(const bf16 *qn, int64_t ldq, const bf16 *wuk,
                                                     int r, bf16 *qlat, int64_t ldo,
                                                     int64_t head_stride, int B) {
  constexpr int WP = AB_N + 8;  // LDS row pitch (elements)
  __shared__ __attribute__((aligned(16))) bf16 Ws[DN * WP];
  const int h = blockIdx.x, n0 = blockIdx.y * AB_N, b0 = blockIdx.z * AB_M;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // stage W_uk_h[:, n0 .. n0 + 127]
  for (int c = tid; c < DN * (AB_N / 8); c += 256) {
    const int k = c / (AB_N / 8), cc = (c % (AB_N / 8)) * 8;
    const int n = n0 + cc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < r) v = *reinterpret_cast<const uint4 *>(wuk + ((int64_t)h * DN + k) * r + n);
    *reinterpret_cast<uint4 *>(&Ws[k * WP + cc]) = v;
  }
  // A fragments: row b = b0 + 32 (wave & 1) + l32, k = 16 f + 8 g .. + 7
  const int bm = b0 + 32 * (wave & 1) + l32;
  bf16x8 af[DN / 16];
#pragma unroll
  for (int f = 0; f < DN / 16; ++f) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (bm < B) v = *reinterpret_cast<const uint4 *>(qn + (int64_t)bm * ldq + (int64_t)h * DN + 16 * f + 8 * g);
    af[f] = __builtin_bit_cast(bf16x8, v);
  }
  __syncthreads();
  // this wave: rows 32 (wave & 1) .., columns 64 (wave >> 1) + 32 t, t < 2
  const int s16 = lane & 15;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nb = 64 * (wave >> 1) + 32 * t;
    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int f = 0; f < DN / 16; ++f) {
      const bf16 *p = &Ws[(16 * f + 8 * g + (s16 >> 2)) * WP + nb + (lane & 16) + 4 * (s16 & 3)];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p + 4 * WP));
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[f], bfr, acc, 0, 0, 0);
    }
    const int n = n0 + nb + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int bb = b0 + 32 * (wave & 1) + acc_row(e, lane);
      if (bb < B && n < r) qlat[(int64_t)bb * ldo + (int64_t)h * head_stride + n] = (bf16)acc[e];
    }
  }
}

template <typename T, int R, int DR>
hipError_t launch_t(const DecodeAttnArgs &a, hipStream_t st) {
  dim3 grid(a.n_blocks * ((a.H + HPB - 1) / HPB));
  hipLaunchKernelGGL((decode_attn_kernel<T, R, DR>), grid, dim3(DTHREADS), 0, st, a);
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_merge_t(const DecodeAttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((decode_merge_kernel<T, R>), dim3(a.B, (a.H + HPW - 1) / HPW),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// Row ranges of a decode step: one workgroup per (range, group of 128 query
// heads) fills the 256 CUs once, so with q_len tokens (q_len head groups at
// 128 heads) the rows are cut into 256 / q_len ranges.
int decode_blocks(int q_len) { return q_len > 1 ? std::max(1, 256 / q_len) : 256; }

hipError_t launch_decode_attention(int dtype, int r, int dr, const DecodeAttnArgs &a,
                                   hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
#define MLA_DEC_CASE(R_, DR_)                                                        \
  if (r == R_ && dr == DR_)                                                          \
    return dtype == BF16 ? launch_t<bf16, R_, DR_>(a, st) : launch_t<float, R_, DR_>(a, st);
  MLA_DEC_CASE(16, 8)
  MLA_DEC_CASE(128, 32)
  // fp32 at the V3 latent width would need more LDS than a CU has; the host
  // rejects it before launching
  if (r == 512 && dr == 64 && dtype == BF16) return launch_t<bf16, 512, 64>(a, st);
#undef MLA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_absorb(int dtype, int dn, int r, int H, int B, const void *qn, int64_t ldq,
                         const void *wuk, void *qlat, int64_t ldo, int64_t head_stride,
                         hipStream_t st) {
  if (dtype != BF16 || dn != 128 || r % 8 != 0) return hipErrorInvalidValue;
  if (B <= 0) return hipSuccess;
  dim3 grid(H, (r + AB_N - 1) / AB_N, (B + AB_M - 1) / AB_M);
  hipLaunchKernelGGL(absorb_kernel<128>, grid, dim3(256), 0, st, (const bf16 *)qn, ldq,
                     (const bf16 *)wuk, r, (bf16 *)qlat, ldo, head_stride, B);
  return hipGetLastError();
}

hipError_t launch_decode_merge(int dtype, int r, const DecodeAttnArgs &a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  if (a.n_blocks + 1 > MERGE_MAXP) return hipErrorInvalidValue;  // piece weights must fit LDS
#define MLA_MERGE_CASE(R_)                                                           \
  if (r == R_) return dtype == BF16 ? launch_merge_t<bf16, R_>(a, st) : launch_merge_t<float, R_>(a, st);
  MLA_MERGE_CASE(16)
  MLA_MERGE_CASE(128)
  if (r == 512 && dtype == BF16) return launch_merge_t<bf16, 512>(a, st);
#undef MLA_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
