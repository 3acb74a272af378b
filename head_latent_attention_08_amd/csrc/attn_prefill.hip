// Causal flash-style prefill attention for MLA heads (gfx950).
//
// Per (batch b, head h): Q = [q_nope_h ‖ q_pe_h] (d_n + d_r wide), K = [k_nope_h ‖
// k_pe] with k_pe shared by all heads, V = v_h (d_v wide); o = softmax(scale Q
// K^T, keys j <= query i) V.  Following the MLA listing of "The Evolving
// Transformer -- DeepSeek V2 & V3" (section 01), with the score matrix never
// written out: keys stream through LDS in tiles and the softmax is kept online
// in fp32 (running max and sum per query, exp2 domain).
//
// Work split: a 256-thread workgroup owns 128 queries of one (b, h); each
// wave owns 32 of them.  A wave computes S^T = K Q^T on 32x32 MFMA tiles
// (keys on the M side, its queries on the N side), so every lane holds scores
// of a single query: the row max needs one cross-lane swap (lane l and l^32)
// and the rescale of the output accumulator is a per-lane multiply.  The
// probabilities stay in registers and feed O^T += V^T P^T directly as the B
// operand; V arrives channel-major ([d][key], written that way by the kv
// up-projection) and is stored to LDS with the middle two 4-key quads of
// every 16-key group swapped, so the eight keys a lane's A operand needs
// (4g..4g+3 and 8+4g..8+4g+3) are one 16-byte read.
//
// Keys (and, for bf16, V^T) stream in tiles of 32 through three LDS stages,
// copied global -> LDS two tiles ahead, one barrier per tile.  Iteration t
// finishes tile t and computes tile t+1's scores; before its barrier a wave
// waits for every copy the next iteration reads (tile t+2's keys included,
// which it issued itself), leaving only its V^T copies of tile t+2 in
// flight.  The softmax keeps a stale running max until a new score exceeds
// it by more than 2^8 (exp2 domain): the probabilities then stay below 256,
// exact in fp32, and the output accumulator is rescaled only on those tiles.
// The score scale folds into the exponent's FMA.
//
// Order: all query tiles of a (b, h) run on one XCD (workgroup ids go to the
// eight XCDs round-robin), so the K/V of a head are fetched from HBM about
// once and then served from that XCD's L2.  An XCD takes its heads two at a
// time, the two heads' query tiles interleaved longest first: with one head
// at a time the longest tiles of the last heads started near the end and ran
// on with most slots already idle (6% longer at S = 4096, 128 heads).

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int BKV = 32;

// s_waitcnt immediate: at most n vector-memory operations of this wave
// outstanding (gfx9 encoding; expcnt and lgkmcnt left open)
#define ATT_VMCNT(n) ((((n) & 15)) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.0f;

template <typename T, int DN, int DR, int DV, int NW>
struct AttnCfg {
  using MF = Mfma32<T>;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int DQK = DN + DR;
  static constexpr int DQKP = (DQK + MF::KSTEP - 1) / MF::KSTEP * MF::KSTEP;
  static constexpr int DVP = (DV + 31) / 32 * 32;
  static constexpr int KPITCH = DQKP + VEC;
  static constexpr int VPITCH = BKV + VEC;
  static constexpr int KSTAGE = BKV * KPITCH;
  static constexpr int VSTAGE = DVP * VPITCH;
  static constexpr int NQF = DQKP / MF::KSTEP;
  static constexpr int NDT = DVP / 32;
  static constexpr int CPRK = DQKP / VEC;        // 16-byte chunks per K row
  static constexpr int CPRV = BKV / VEC;         // 16-byte chunks per V^T row
  static constexpr int KCH = (BKV * CPRK + 255) / 256;
  static constexpr int VCH = (DV * CPRV + 255) / 256;
  // K stage in LDS, filled by 1 KB copy blocks: k_nope rows (pitch KNP), then
  // k_pe rows (pitch KPP, padded to whole query fragments)
  static constexpr int ES = sizeof(T);
  static constexpr int NQN = DN / MF::KSTEP;   // query fragments over k_nope
  static constexpr int KNP = DN + VEC;
  static constexpr int KPP = (DQKP - DN) + VEC;
  static constexpr int NKN = (BKV * KNP * ES + 1023) / 1024;
  static constexpr int NKP = (BKV * KPP * ES + 1023) / 1024;
  static constexpr int KSTAGEB = (NKN + NKP) * 1024;
  static constexpr int NKPW = (NKN + NKP + NW - 1) / NW;  // copy blocks per wave (at most)
  // V^T stage copied straight from global memory (bf16, 32 keys = 64-byte
  // rows): DVP rows in 1 KB blocks of 16
  static constexpr int NVB = DVP / 16;
  static constexpr int NVPW = (NVB + NW - 1) / NW;
};

// Key order inside each 16-key group of a tile as seen by the score MFMA when
// V^T is copied verbatim: the lane feeding score row x reads key pk16(x)
// (bits 2 and 3 of x swapped).  A lane of half g holds score rows
// 16u + 8a + 4g + c (a < 2, c < 4) of slice u, i.e. keys 16u + 8g + 4a + c:
// the eight k slots of its probability operand are eight consecutive keys,
// which the V^T operand reads as one 16-byte chunk of its row.
__device__ inline int pk16(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <typename T>
__device__ inline uint4 ld16(const T *p) { return *reinterpret_cast<const uint4 *>(p); }

// VD: bf16 with S a multiple of 8 -- V^T tiles are copied global -> LDS by
// the same copy instructions as the keys (no staging registers, no LDS
// stores), with the score MFMA reading keys in pk16 order.  Otherwise V^T
// is staged through registers and stored to LDS with two quads swapped.
template <typename T, int DN, int DR, int DV, bool VD, int NW, bool VARLEN>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(PrefillAttnArgs a) {
  using C = AttnCfg<T, DN, DR, DV, NW>;
  constexpr int BQ = 32 * NW;  // queries per workgroup: 32 per wave
  using MF = typename C::MF;
  constexpr int VEC = C::VEC, DQK = C::DQK, KPITCH = C::KPITCH, VPITCH = C::VPITCH,
                NQF = C::NQF, NDT = C::NDT, DVP = C::DVP, CPRK = C::CPRK, CPRV = C::CPRV,
                DQKP = C::DQKP, ES = C::ES, NQN = C::NQN, KNP = C::KNP, KPP = C::KPP,
                NKN = C::NKN, NKP = C::NKP, KSTAGEB = C::KSTAGEB, NKPW = C::NKPW,
                KCH = C::KCH, VCH = C::VCH, KSTAGE = C::KSTAGE, VSTAGE = C::VSTAGE,
                NVB = C::NVB, NVPW = C::NVPW;
  static_assert(!VD || (sizeof(T) == 2 && BKV == 32), "verbatim V^T copies need bf16 tiles of 32");
  static_assert(VD || NW == 4, "the register-staged V^T path assumes 256 threads");
  __shared__ __attribute__((aligned(1024))) char Kl[3 * KSTAGEB];
  __shared__ __attribute__((aligned(1024))) char Vl[VD ? 3 * NVB * 1024 : 16];
  __shared__ __attribute__((aligned(16))) T Vt[VD ? VEC : 3 * VSTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: feeds M0
  const int g = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H;
  // keys: the queries' own tokens, or (key ranges) a key stream of its own
  const int SK = VARLEN ? a.Sk : S;
  const int nq = (S + BQ - 1) / BQ;
  const int P = a.B * H;
  const int w = blockIdx.x;
  int pair, qt;
  if ((P & 15) == 0) {
    // the (b, h) of an XCD in pairs, the query tiles of a pair interleaved
    // longest first
    const int local = w >> 3;
    const int grp = local / (2 * nq), r = local - grp * (2 * nq);
    pair = (w & 7) * (P >> 3) + 2 * grp + (r & 1);
    qt = nq - 1 - (r >> 1);
  } else if ((P & 7) == 0) {
    const int local = w >> 3;
    pair = (w & 7) * (P >> 3) + local / nq;
    qt = nq - 1 - local % nq;
  } else {
    pair = w / nq;
    qt = nq - 1 - w % nq;
  }
  const int b = pair / H, h = pair - b * H;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;
  const int iq = qw0 + l32;  // this lane's query

  const int64_t bh = (int64_t)b * H + h;
  const T *qp = reinterpret_cast<const T *>(a.q) + bh * S * DQK;
  const T *kn = reinterpret_cast<const T *>(a.k_nope) + bh * SK * DN;
  const T *kpe = reinterpret_cast<const T *>(a.k_pe) + (int64_t)b * SK * a.ld_kpe;
  const T *vt = reinterpret_cast<const T *>(a.vt) + bh * DV * SK;

  if constexpr (DVP > DV && !VD) {
    for (int i = tid; i < (DVP - DV) * VPITCH; i += 256) {
      Vt[DV * VPITCH + i] = from_f32<T>(0.f);
      Vt[VSTAGE + DV * VPITCH + i] = from_f32<T>(0.f);
      Vt[2 * VSTAGE + DV * VPITCH + i] = from_f32<T>(0.f);
    }
  }

  // this lane's query fragments, kept in registers for the whole key loop
  typename MF::frag qf[NQF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    const int c = f * MF::KSTEP + g * MF::KPL;
    if constexpr (MF::KPL == 1) {
      qf[f] = (iq < S && c < DQK) ? to_f32(qp[(int64_t)iq * DQK + c]) : 0.f;
    } else {
      if (iq < S && c < DQK) {
        uint4 v = ld16(qp + (int64_t)iq * DQK + c);
        qf[f] = *reinterpret_cast<typename MF::frag *>(&v);
      } else {
#pragma unroll
        for (int e = 0; e < MF::KPL; ++e) qf[f][e] = from_f32<T>(0.f);
      }
    }
  }

  // K tiles are copied from global memory straight into LDS
  // (global_load_lds_dwordx4, 16 bytes a lane into consecutive LDS bytes of a
  // 1 KB block).  This wave copies blocks wave, wave + NW, ..; a lane's row
  // and byte column in its block are fixed for the whole loop (padding
  // lanes copy the tile's first chunk: finite values that only meet zero
  // query columns), the tile base is a scalar, and rows past the end of the
  // sequence (last tile only, masked keys) repeat the last row.
  int drow[NKPW], dcb[NKPW];
#pragma unroll
  for (int k = 0; k < NKPW; ++k) {
    const int blk = wave + NW * k;
    drow[k] = 0;
    dcb[k] = 0;
    if (blk < NKN) {
      const int o = blk * 1024 + lane * 16, row = o / (KNP * ES), cb = o - row * (KNP * ES);
      if (row < BKV && cb < DN * ES) { drow[k] = row; dcb[k] = cb; }
    } else if (blk < NKN + NKP) {
      const int o = (blk - NKN) * 1024 + lane * 16, row = o / (KPP * ES), cb = o - row * (KPP * ES);
      if (row < BKV && cb < DR * ES) { drow[k] = row; dcb[k] = cb; }
    }
  }
  const uint32_t lds_k = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)Kl;
  // Per copy k of this wave: its block's source rows (k_nope, or the shared
  // k_pe) and their pitch, and this lane's byte offset from the tile's first
  // row.  Every wave issues the first NKALL copies of a tile, the waves with
  // a block left one more; a tile running past the last key (only the last
  // tile can) clamps the rows, every other tile takes the fixed offsets.
  const T *ksrc[NKPW];
  int kpb[NKPW];
  uint32_t koff[NKPW];
#pragma unroll
  for (int k = 0; k < NKPW; ++k) {
    const bool nope = wave + NW * k < NKN;
    ksrc[k] = nope ? kn : kpe;
    kpb[k] = nope ? DN * ES : a.ld_kpe * ES;
    koff[k] = (uint32_t)(drow[k] * kpb[k] + dcb[k]);
  }
  constexpr int NKALL = (NKN + NKP) / NW;
  const bool kmore = wave + NW * NKALL < NKN + NKP;
#define ATT_KCOPY(STG, J0, k, OFF)                                                      \
  do {                                                                                  \
    const char *src_ = reinterpret_cast<const char *>(ksrc[k]) + (int64_t)(J0) * kpb[k]; \
    const uint32_t m0_ = lds_k + (STG) * KSTAGEB + (wave + NW * (k)) * 1024;            \
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"                   \
                 :: "v"(OFF), "s"(src_), "s"(m0_) : "memory", "m0");                    \
  } while (0)
#define ATT_KDMA(STG, J0)                                                               \
  do {                                                                                  \
    const int j0_ = (J0);                                                               \
    if (j0_ + BKV <= SK) {                                                              \
      _Pragma("unroll") for (int k = 0; k < NKPW; ++k)                                  \
        if (k < NKALL || kmore) ATT_KCOPY(STG, j0_, k, koff[k]);                        \
    } else {                                                                            \
      const int lim_ = SK - 1 - j0_;                                                    \
      _Pragma("unroll") for (int k = 0; k < NKPW; ++k)                                  \
        if (k < NKALL || kmore)                                                         \
          ATT_KCOPY(STG, j0_, k, (uint32_t)(min(drow[k], lim_) * kpb[k] + dcb[k]));     \
    }                                                                                   \
  } while (0)

  // VD: V^T tile copies.  Block vb = wave + NW k holds rows 16 vb .. + 15 (64
  // bytes = 32 keys each); lane l fills row 16 vb + l/4 at position l%4,
  // which holds logical 16-byte chunk (l%4) ^ (row/4 % 4) (conflict-free
  // 16-byte reads of 16 consecutive rows).  Rows past DV repeat row 0 (their
  // output channels are never stored); chunks past the sequence repeat the
  // last one (masked keys).
  const T *vt_bh = reinterpret_cast<const T *>(a.vt) + bh * DV * SK;
  int vrow[NVPW], vch[NVPW];
#pragma unroll
  for (int k = 0; k < NVPW; ++k) {
    const int row = 16 * (wave + NW * k) + (lane >> 2);
    vrow[k] = row < DV ? row : 0;
    vch[k] = (lane & 3) ^ ((row >> 2) & 3);
  }
  const uint32_t lds_v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)Vl;
  // this lane's byte offset from the tile's first key in a whole tile
  uint32_t voff[NVPW];
#pragma unroll
  for (int k = 0; k < NVPW; ++k) voff[k] = (uint32_t)((vrow[k] * SK + 8 * vch[k]) * ES);
#define ATT_VCOPY(STG, SRC, k, OFF)                                                     \
  do {                                                                                  \
    const uint32_t m0_ = lds_v + (STG) * (NVB * 1024) + (wave + NW * (k)) * 1024;       \
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"                   \
                 :: "v"(OFF), "s"(SRC), "s"(m0_) : "memory", "m0");                     \
  } while (0)
#define ATT_VDMA(STG, J0)                                                               \
  do {                                                                                  \
    const int j0_ = (J0);                                                               \
    if (j0_ + BKV <= SK) {                                                              \
      const T *src_ = vt_bh + j0_;                                                      \
      _Pragma("unroll") for (int k = 0; k < NVPW; ++k)                                  \
        if (NVB % NW == 0 || wave + NW * k < NVB) ATT_VCOPY(STG, src_, k, voff[k]);     \
    } else {                                                                            \
      _Pragma("unroll") for (int k = 0; k < NVPW; ++k)                                  \
        if (NVB % NW == 0 || wave + NW * k < NVB)                                       \
          ATT_VCOPY(STG, vt_bh, k, (uint32_t)((vrow[k] * SK + min(j0_ + 8 * vch[k], SK - 8)) * ES)); \
    }                                                                                   \
  } while (0)
  // V^T copies of this wave per tile (0 .. NVPW), for the wait counts
  const int nvcopy = (NVB - wave + NW - 1) / NW;

  // register staging of one V^T tile (plain code, not lambdas: the staging
  // registers must not end up in scratch memory)
  uint4 rv[VCH];
  const bool v_whole = __builtin_amdgcn_readfirstlane(SK % VEC == 0 && SK >= VEC);
#define ATT_FETCH(J0)                                                               \
  do {                                                                              \
    const int j0_ = (J0);                                                           \
    _Pragma("unroll") for (int i = 0; i < VCH; ++i) {                               \
      const int c = min(tid + 256 * i, DV * CPRV - 1);                              \
      const int d = c / CPRV, jc = (c - d * CPRV) * VEC;                            \
      const int j = j0_ + jc;                                                       \
      uint4 v;                                                                      \
      if (v_whole) {                                                                \
        /* S is a multiple of VEC: a chunk is wholly inside or wholly past */       \
        /* the end; past-the-end chunks repeat the last one (masked keys) */        \
        v = ld16(vt + (int64_t)d * SK + min(j, SK - VEC));                          \
      } else {                                                                      \
        const T *src = vt + (int64_t)d * SK + j;                                    \
        T e[VEC];                                                                   \
        _Pragma("unroll") for (int k = 0; k < VEC; ++k)                             \
            e[k] = (j + k < SK) ? src[k] : from_f32<T>(0.f);                        \
        v = *reinterpret_cast<const uint4 *>(e);                                    \
      }                                                                             \
      rv[i] = v;                                                                    \
    }                                                                               \
  } while (0)
#define ATT_STASH(STAGE)                                                            \
  do {                                                                              \
    T *vs_ = Vt + (STAGE) * VSTAGE;                                                 \
    _Pragma("unroll") for (int i = 0; i < VCH; ++i) {                               \
      const int c = tid + 256 * i;                                                  \
      if (c < DV * CPRV) {                                                          \
        const int d = c / CPRV, jc = (c - d * CPRV) * VEC;                          \
        if constexpr (MF::KPL > 1) {                                                \
          /* keys 8h..8h+7 of a 16-key group: quads to positions 4h and 4h+8 */    \
          T *dst_ = &vs_[d * VPITCH + (jc & ~15) + ((jc >> 1) & 4)];                \
          *reinterpret_cast<uint2 *>(dst_) = make_uint2(rv[i].x, rv[i].y);          \
          *reinterpret_cast<uint2 *>(dst_ + 8) = make_uint2(rv[i].z, rv[i].w);      \
        } else {                                                                    \
          *reinterpret_cast<uint4 *>(&vs_[d * VPITCH + jc]) = rv[i];                \
        }                                                                           \
      }                                                                             \
    }                                                                               \
  } while (0)

  f32x16 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * LOG2E;

  // Key tiles t = 0.. start at key jb.  Causal: keys 0..iq, jb = 0.  Key
  // ranges: query iq takes keys kv_lo[iq] .. kv_hi[iq], both non-decreasing
  // along the queries, so the block needs the tiles from its first query's
  // kv_lo to its last query's kv_hi; a lane masks the keys outside its own
  // range.
  const int iqc = min(iq, S - 1);
  const int key_lo = VARLEN ? a.kv_lo[iqc] : 0;
  const int key_hi = VARLEN ? a.kv_hi[iqc] : iq;
  const int jb = VARLEN ? a.kv_lo[q0] / BKV * BKV : 0;
  const int kv_end = VARLEN ? a.kv_hi[min(S, q0 + BQ) - 1] + 1 : min(S, q0 + BQ);
  const int ntiles = (kv_end + BKV - 1) / BKV - jb / BKV;
  // this wave's last tile (a wave with no query left needs none)
  const int tw = VARLEN ? (qw0 < S ? a.kv_hi[min(qw0 + 31, S - 1)] / BKV - jb / BKV : -1)
                        : qw0 / BKV - jb / BKV;

  // fragment f of this lane's key row in the K stage starting at byte KB:
  // k_nope region for f < NQN, k_pe region after it
  const int kr = VD ? pk16(l32) : l32;  // key row this lane feeds to the score MFMA
#define ATT_KFRAG(KB, f)                                                              \
  (*reinterpret_cast<const typename MF::frag *>(                                      \
      (f) < NQN ? reinterpret_cast<const T *>(KB) + kr * KNP + (f) * MF::KSTEP + g * MF::KPL \
                : reinterpret_cast<const T *>((KB) + NKN * 1024) + kr * KPP +         \
                      ((f) - NQN) * MF::KSTEP + g * MF::KPL))
  // S^T of key tile at stage byte base KB for this wave's queries
#define ATT_QK(ST, KB)                                                                \
  do {                                                                                \
    _Pragma("unroll") for (int r = 0; r < 16; ++r) ST[r] = 0.f;                       \
    _Pragma("unroll") for (int f = 0; f < NQF; ++f) {                                 \
      const typename MF::frag kf_ = ATT_KFRAG(KB, f);                                 \
      ST = MF::mma(kf_, qf[f], ST);                                                   \
    }                                                                                 \
  } while (0)
  // Pipeline over key tiles: tile t sits in LDS stage t % 3.  Iteration t
  // starts the copy of tile t+2's keys into the stage tile t-1 used, then
  // finishes tile t (softmax, O^T += V^T P^T) while the MFMAs of tile t+1's
  // scores run underneath the exponentials, and stores tile t+2's V^T
  // (loaded into registers one iteration earlier).
  if constexpr (VD) {
    ATT_KDMA(0, jb);
    ATT_VDMA(0, jb);
    if (ntiles > 1) {
      ATT_KDMA(1, jb + BKV);
      ATT_VDMA(1, jb + BKV);
    }
  } else {
    ATT_KDMA(0, jb);
    ATT_FETCH(jb);
    ATT_STASH(0);
    if (ntiles > 1) {
      ATT_KDMA(1, jb + BKV);
      ATT_FETCH(jb + BKV);
      ATT_STASH(1);
    }
    if (ntiles > 2) ATT_FETCH(jb + 2 * BKV);
  }
  __builtin_amdgcn_s_waitcnt(ATT_VMCNT(0));
  __syncthreads();
  f32x16 s_cur;
  ATT_QK(s_cur, Kl);
  int rd = 0;  // stage of tile t
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = jb + t * BKV;
    const int rn = rd == 2 ? 0 : rd + 1;   // stage of tile t + 1
    const int rw = rd == 0 ? 2 : rd - 1;   // stage of tile t + 2 (held tile t - 1)
    if (t + 2 < ntiles) {
      ATT_KDMA(rw, jb + (t + 2) * BKV);
      if constexpr (VD) ATT_VDMA(rw, jb + (t + 2) * BKV);
    }
    if (t <= tw) {
      // The compute part of an iteration runs at raised wave priority: of the
      // two waves sharing a SIMD, the one issuing MFMAs and exponentials wins
      // issue over the other's copy, wait and mask work (4% faster).
      __builtin_amdgcn_s_setprio(1);
      // V^T fragments of tile t, read now so that they have landed by the
      // time the PV MFMAs issue (bf16; the fp32 path reads them in place)
      const T *vs = Vt + rd * VSTAGE;
      typename MF::frag vpre[MF::KPL > 1 ? 2 : 1][NDT];
      if constexpr (VD) {
        // rows d*32 + l32 of the verbatim stage; keys 16u + 8g .. +7 are
        // logical chunk 2u + g
        const T *vl = reinterpret_cast<const T *>(Vl + __builtin_amdgcn_readfirstlane(rd * NVB * 1024));
        const int sw = (l32 >> 2) & 3;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int d = 0; d < NDT; ++d)
            vpre[u][d] = *reinterpret_cast<const typename MF::frag *>(
                vl + (d * 32 + l32) * BKV + (((2 * u + g) ^ sw) << 3));
      } else if constexpr (MF::KPL > 1) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int d = 0; d < NDT; ++d) {
            // k slots e = 0..7 hold keys (e/4)*8 + g*4 + e%4 of 16-key slice u,
            // which the stash laid out contiguously at u*16 + g*8
            const T *row = &vs[(d * 32 + l32) * VPITCH];
            vpre[u][d] = *reinterpret_cast<const typename MF::frag *>(row + u * 16 + g * 8);
          }
      }
      // the first three key fragments of tile t+1, read before the mask and
      // max so that the score MFMAs below find them landed; each MFMA then
      // reads the fragment three ahead (one ahead left every MFMA waiting
      // out most of an LDS read's latency: 5% slower overall)
      const char *ksn = Kl + __builtin_amdgcn_readfirstlane(rn * KSTAGEB);
      typename MF::frag kq0 = ATT_KFRAG(ksn, 0);
      typename MF::frag kq1 = ATT_KFRAG(ksn, NQF > 1 ? 1 : 0);
      typename MF::frag kq2 = ATT_KFRAG(ksn, NQF > 2 ? 2 : 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (VARLEN) {
        // keys outside this query's range
        if (j0 < key_lo || j0 + BKV - 1 > key_hi) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = j0 + (VD ? pk16(acc_row(r, lane)) : acc_row(r, lane));
            if (kj < key_lo || kj > key_hi) s_cur[r] = -INFINITY;
          }
        }
      } else if (t == tw) {
        // causal mask on the diagonal tile only; key j0 + acc_row(r) is
        // masked when acc_row(r) exceeds iq - j0
        if constexpr (VD) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (pk16(acc_row(r, lane)) > iq - j0) s_cur[r] = -INFINITY;
        } else {
          const int lim = iq - j0 - g * 4;  // acc_row(r) = (r/4)*8 + g*4 + r%4
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((r >> 2) * 8 + (r & 3) > lim) s_cur[r] = -INFINITY;
        }
      }
      float mx = s_cur[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
      mx = half_swap_max(mx);
      // rescale only when the max grew past the allowance (or on first use)
      const bool need = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f((m_run - mx) * sl2) : 1.0f;
        if (need) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < NDT; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      // hardware exp2: arguments are <= 2^8 above zero, and large negative
      // ones (masked keys) may flush to 0
      const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
      // Tile t+1's score MFMAs, each followed by a share of tile t's
      // exponentials: independent work the wave issues while the MFMA runs.
      // They run even when the wave needs no tile t+1 (its diagonal tile or
      // the last tile): the stage then holds stale but in-bounds data and
      // the result is dropped; a branch here would let the compiler hoist
      // the exponentials out of the interleaving.
      f32x16 s_nxt;
      {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_nxt[r] = 0.f;
        // the fences keep the issue order as written: read fragment f+3,
        // MFMA f, then VALU work that does not depend on it
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          typename MF::frag kn_ = kq0;
          if (f + 3 < NQF) kn_ = ATT_KFRAG(ksn, f + 3);
          __builtin_amdgcn_sched_barrier(0);
          s_nxt = MF::mma(kq0, qf[f], s_nxt);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = f * 16 / NQF; r < (f + 1) * 16 / NQF; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(s_cur[r], sl2, neg));
            s_cur[r] = pr;
            if constexpr (MF::KPL == 1) l_run += pr;
          }
          __builtin_amdgcn_sched_barrier(0);
          kq0 = kq1;
          kq1 = kq2;
          kq2 = kn_;
        }
      }
      // O^T += V^T P^T with P^T taken from the score accumulators in place
#pragma unroll
      for (int u = 0; u < 16 / MF::KPL; ++u) {
        typename MF::frag pf;
        if constexpr (MF::KPL == 1) {
          pf = s_cur[u];
        } else {
#pragma unroll
          for (int e = 0; e < MF::KPL; ++e) pf[e] = from_f32<T>(s_cur[u * MF::KPL + e]);
          // the row sum takes the bf16 probabilities the PV product uses, two
          // at a time (dot with (1, 1))
          const bf16x2 one2 = {from_f32<T>(1.f), from_f32<T>(1.f)};
#pragma unroll
          for (int e = 0; e < MF::KPL; e += 2) {
            const bf16x2 p2 = {pf[e], pf[e + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, one2, l_run, false);
          }
        }
#pragma unroll
        for (int d = 0; d < NDT; ++d) {
          const T *row = &vs[(d * 32 + l32) * VPITCH];
          typename MF::frag vf;
          if constexpr (MF::KPL == 1) vf = to_f32(row[acc_row(u, lane)]);
          else vf = vpre[u][d];
          o[d] = MF::mma(vf, pf, o[d]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      s_cur = s_nxt;
    }
    if constexpr (VD) {
      // The next iteration reads tile t+1's V^T and tile t+2's keys (its
      // next-tile scores).  This iteration issued tile t+2's key copies
      // before its V^T copies, so once at most this wave's V^T copies of
      // tile t+2 are outstanding, everything the next iteration reads from
      // this wave has landed; the barrier publishes every wave's.
      if (t + 2 < ntiles) {
        if (nvcopy == NVPW) __builtin_amdgcn_s_waitcnt(ATT_VMCNT(NVPW));
        else if (nvcopy == NVPW - 1) __builtin_amdgcn_s_waitcnt(ATT_VMCNT(NVPW - 1));
        else __builtin_amdgcn_s_waitcnt(ATT_VMCNT(0));
      } else {
        __builtin_amdgcn_s_waitcnt(ATT_VMCNT(0));
      }
    } else {
      if (t + 2 < ntiles) {
        ATT_STASH(rw);
        if (t + 3 < ntiles) ATT_FETCH(jb + (t + 3) * BKV);
      }
      // this wave's key copies of tile t+2 have landed (only the V^T loads of
      // tile t+3, issued after them, may still be in flight); the barrier
      // publishes every wave's copies and stores
      if (t + 3 < ntiles && v_whole) __builtin_amdgcn_s_waitcnt(ATT_VMCNT(VCH));
      else __builtin_amdgcn_s_waitcnt(ATT_VMCNT(0));
    }
    __syncthreads();
    rd = rn;
  }
#undef ATT_KFRAG
#undef ATT_KDMA
#undef ATT_KCOPY
#undef ATT_QK
#undef ATT_FETCH
#undef ATT_STASH
#undef ATT_VDMA
#undef ATT_VCOPY

  // normalise and store o[b, i, h, d]
  const float l_tot = half_swap_sum(l_run);
  // invalid sequence offsets: every output is NaN
  const float inv = (VARLEN && a.valid && a.valid[iqc] == 0) ? __builtin_nanf("") : 1.0f / l_tot;
  if (iq < S) {
    T *op = reinterpret_cast<T *>(a.o) + ((int64_t)b * S + iq) * (int64_t)H * DV + (int64_t)h * DV;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int dd = d * 32 + acc_row(r, lane);
        if (dd + 4 <= DV) {
          T v4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = from_f32<T>(o[d][r + e] * inv);
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint2 *>(op + dd) = *reinterpret_cast<const uint2 *>(v4);
          } else {
            *reinterpret_cast<uint4 *>(op + dd) = *reinterpret_cast<const uint4 *>(v4);
          }
        }
      }
  }
}

// Waves per workgroup on the bf16 copy path.  Eight waves over 256 queries
// halve the copies per key tile but run 9% slower than two independent
// 4-wave workgroups per CU, whose phases drift apart so that one's softmax
// overlaps the other's MFMAs.
constexpr int ATT_VD_WAVES = 4;

template <typename T, int DN, int DR, int DV>
hipError_t launch_t(const PrefillAttnArgs &a, hipStream_t st) {
  const bool varlen = a.kv_lo != nullptr;
  const int sk = varlen ? a.Sk : a.S;
  if constexpr (sizeof(T) == 2) {
    if (sk % 8 == 0) {
      constexpr int NW = ATT_VD_WAVES;
      dim3 grid((a.S + 32 * NW - 1) / (32 * NW) * a.H * a.B);
      if (varlen)
        hipLaunchKernelGGL((prefill_attn_kernel<T, DN, DR, DV, true, NW, true>), grid, dim3(64 * NW), 0,
                           st, a);
      else
        hipLaunchKernelGGL((prefill_attn_kernel<T, DN, DR, DV, true, NW, false>), grid, dim3(64 * NW), 0,
                           st, a);
      return hipGetLastError();
    }
  }
  dim3 grid((a.S + 127) / 128 * a.H * a.B);
  if (varlen)
    hipLaunchKernelGGL((prefill_attn_kernel<T, DN, DR, DV, false, 4, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<T, DN, DR, DV, false, 4, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attention(int dtype, int dn, int dr, int dv, const PrefillAttnArgs &a,
                                    hipStream_t st) {
  if (a.S <= 0 || a.B <= 0) return hipSuccess;
#define MLA_ATTN_CASE(DN_, DR_, DV_)                                              \
  if (dn == DN_ && dr == DR_ && dv == DV_)                                        \
    return dtype == BF16 ? launch_t<bf16, DN_, DR_, DV_>(a, st)                   \
                         : launch_t<float, DN_, DR_, DV_>(a, st);
  MLA_ATTN_CASE(16, 8, 16)
  MLA_ATTN_CASE(64, 32, 64)
  MLA_ATTN_CASE(128, 64, 128)
#undef MLA_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
