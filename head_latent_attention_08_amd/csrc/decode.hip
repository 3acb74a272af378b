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
// Work split: the rows of all sequences (lens[b] + 1 each, the new token
// included) are laid end to end and cut into n_blocks equal ranges, so long
// and short sequences load the GPU evenly.  Each range is processed by one
// workgroup per group of 64 heads; the workgroups of a range are numbered so
// they land on the same XCD at the same time (workgroup ids go to the eight
// XCDs round-robin) and the second read of every cache tile hits that XCD's
// L2.  A range that spans sequence boundaries yields one partial
// (unnormalised o_lat, running max, running sum) per sequence piece, in slot
// (range + b) -- unique because range and sequence indices both rise along
// the flattened rows.  A merge kernel combines the pieces of each sequence
// with log-sum-exp weights.
//
// Inside a workgroup: four waves, 16 heads each, on 16x16x32 MFMAs.  A wave
// computes S^T = C Q^T (16 cache rows x 16 heads per tile, K = 576), keeps the
// softmax online per head, and accumulates O^T += C^T P^T with P^T taken from
// the score accumulators in place.  The C^T operand comes straight from the
// row-major cache tile through the 16-bit transposing LDS read: within each
// 16-lane group, lane i receives element i % 4 of the 8-byte chunks
// addressed by lanes 4e + i / 4 (e = 0..3), so pointing lane s at row
// j0 + s / 4, column c0 + 4 (s % 4) hands every lane keys j0..j0+3 of its own
// column c0 + i.  Cache tiles of 32 rows stream through two LDS stages with
// register prefetch of the tile after next; the running max is kept stale
// until a score exceeds it by 2^8, so the accumulators are rarely rescaled.
// Sixteen heads per wave keep the per-lane state (128 accumulators, 72
// registers of queries) well inside the register file; LDS read bandwidth
// (about 215 B/clk per CU measured for 16-byte reads) covers the four waves
// reading every tile.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int TK = 32;   // cache rows per tile
constexpr int HPW = 16;  // heads per wave
constexpr int HPB = 64;  // heads per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.0f;

template <typename T, int R, int DR>
struct DecCfg {
  using MF = Mfma16<T>;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int W = R + DR;
  static constexpr int WP = (W + MF::KSTEP - 1) / MF::KSTEP * MF::KSTEP;
  static constexpr int RP = (R + 15) / 16 * 16;
  static constexpr int CPITCH = (WP > RP ? WP : RP) + VEC;  // 1168 B at V3 sizes
  static constexpr int STAGE = TK * CPITCH;
  static constexpr int NQF = WP / MF::KSTEP;
  static constexpr int NCT = RP / 16;
  static constexpr int CPR = W / VEC;                 // 16-byte chunks per cache row
  static constexpr int NCH = (TK * CPR + 255) / 256;  // staging chunks per thread
};

// Rows of sequence b in the flattened order: lens[b] + 1 for a valid length.
__device__ inline int seq_rows(const int32_t *lens, int b, int64_t cap) {
  const int32_t L = lens[b];
  return (L >= 0 && (int64_t)L < cap) ? L + 1 : 0;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T, int R, int DR>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  using C = DecCfg<T, R, DR>;
  using MF = typename C::MF;
  constexpr int VEC = C::VEC, W = C::W, CPITCH = C::CPITCH, STAGE = C::STAGE, NQF = C::NQF,
                NCT = C::NCT, CPR = C::CPR, NCH = C::NCH;
  __shared__ __attribute__((aligned(16))) T Cs[2 * STAGE];
  extern __shared__ int starts[];  // [B + 1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
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
  const int h = hg * HPB + wave * HPW + l16;
  const bool wave_live = hg * HPB + wave * HPW < H;

  // prefix sums of per-sequence row counts
  for (int b = tid; b < B; b += 256) starts[b + 1] = seq_rows(a.lens, b, a.cap);
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
      const int b = c0 + lane;
      int v = b < B ? starts[b + 1] : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
      }
      if (b < B) starts[b + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (lane == 0) starts[0] = 0;
  }
  __syncthreads();
  const int total = starts[B];
  const int per = (total + a.n_blocks - 1) / a.n_blocks;
  int r0 = blk * per;
  const int r1 = min(r0 + per, total);
  if (r0 >= r1) return;
  int b = 0;
  while (starts[b + 1] <= r0) ++b;  // first sequence holding row r0

  if constexpr (CPITCH - VEC > W) {
    // columns past the row width feed only products with zero queries or
    // output channels >= R; keep them finite
    for (int i = tid; i < 2 * TK; i += 256)
      for (int c = W; c < CPITCH; ++c) Cs[(i / TK) * STAGE + (i % TK) * CPITCH + c] = from_f32<T>(0.f);
  }
  const float sl2 = a.scale * LOG2E;
  const T *cache = reinterpret_cast<const T *>(a.cache);

  uint4 rc[NCH];
#define DEC_FETCH(T0)                                                                \
  do {                                                                               \
    const int t0_ = (T0);                                                            \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                                \
      const int c = tid + 256 * i;                                                   \
      const int jr = c / CPR, cc = (c - jr * CPR) * VEC;                             \
      uint4 v = make_uint4(0, 0, 0, 0);                                              \
      if (c < TK * CPR && t0_ + jr < t_end)                                          \
        v = *reinterpret_cast<const uint4 *>(cb + (int64_t)(t0_ + jr) * W + cc);     \
      rc[i] = v;                                                                     \
    }                                                                                \
  } while (0)
#define DEC_STASH(STG)                                                               \
  do {                                                                               \
    T *cs_ = Cs + (STG) * STAGE;                                                     \
    _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                                \
      const int c = tid + 256 * i;                                                   \
      if (c < TK * CPR) {                                                            \
        const int jr = c / CPR, cc = (c - jr * CPR) * VEC;                           \
        *reinterpret_cast<uint4 *>(&cs_[jr * CPITCH + cc]) = rc[i];                  \
      }                                                                              \
    }                                                                                \
  } while (0)

  while (r0 < r1) {
    const int seg_end = min(r1, starts[b + 1]);
    const int t_begin = r0 - starts[b], t_end = seg_end - starts[b];
    const T *cb = cache + (int64_t)b * a.cap * W;

    // B operand of S^T = C Q^T: lane holds head l16, k values q*KPL.. of each step
    typename MF::frag qf[NQF];
    const T *qp = reinterpret_cast<const T *>(a.q_lat) + ((int64_t)b * H + h) * W;
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      const int c = f * MF::KSTEP + q * MF::KPL;
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
    f32x4 o[NCT];
#pragma unroll
    for (int d = 0; d < NCT; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[d][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int ntiles = (t_end - t_begin + TK - 1) / TK;
    __syncthreads();  // the previous segment's last tile is fully consumed
    DEC_FETCH(t_begin);
    DEC_STASH(0);
    if (ntiles > 1) DEC_FETCH(t_begin + TK);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int t0 = t_begin + it * TK;
      const T *cs = Cs + (it & 1) * STAGE;
      if (wave_live) {
        // S^T for keys 0..15 (s0) and 16..31 (s1) of the tile: lane holds keys
        // q*4 + r (+16), head l16
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NQF; ++f) {
          const int c = f * MF::KSTEP + q * MF::KPL;
          typename MF::frag k0, k1;
          if constexpr (MF::KPL == 1) {
            k0 = to_f32(cs[l16 * CPITCH + c]);
            k1 = to_f32(cs[(16 + l16) * CPITCH + c]);
          } else {
            k0 = *reinterpret_cast<const typename MF::frag *>(&cs[l16 * CPITCH + c]);
            k1 = *reinterpret_cast<const typename MF::frag *>(&cs[(16 + l16) * CPITCH + c]);
          }
          s0 = MF::mma(k0, qf[f], s0);
          s1 = MF::mma(k1, qf[f], s1);
        }
        if (t0 + TK > t_end) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (t0 + q * 4 + r >= t_end) s0[r] = -INFINITY;
            if (t0 + 16 + q * 4 + r >= t_end) s1[r] = -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need =
            mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
        if (__any(need)) {
          const float alpha = need ? exp2f((m_run - mx) * sl2) : 1.0f;
          if (need) m_run = mx;
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < NCT; ++d) o[d] *= alpha;
        }
        const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s0[r] = exp2f(fmaf(s0[r], sl2, neg));
          s1[r] = exp2f(fmaf(s1[r], sl2, neg));
          l_run += s0[r] + s1[r];
        }
        // O^T += C^T P^T: for bf16 one MFMA per 16 latent channels covers all
        // 32 keys; k slots 0..3 are keys q*4 + e, slots 4..7 keys 16 + q*4 + e
        if constexpr (MF::KPL == 1) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float pf = t < 4 ? s0[t] : s1[t - 4];
            const int key = (t < 4 ? 0 : 16) + q * 4 + (t & 3);
#pragma unroll
            for (int d = 0; d < NCT; ++d)
              o[d] = MF::mma(to_f32(cs[key * CPITCH + d * 16 + l16]), pf, o[d]);
          }
        } else {
          typename MF::frag pf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[e] = from_f32<T>(s0[e]);
            pf[4 + e] = from_f32<T>(s1[e]);
          }
          const T *pbase = &cs[(q * 4 + (l16 >> 2)) * CPITCH + 4 * (l16 & 3)];
#pragma unroll
          for (int d = 0; d < NCT; ++d) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(pbase + d * 16));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(pbase + 16 * CPITCH + d * 16));
            const typename MF::frag vf = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[d] = MF::mma(vf, pf, o[d]);
          }
        }
      }
      if (it + 1 < ntiles) {
        DEC_STASH((it + 1) & 1);
        if (it + 2 < ntiles) DEC_FETCH(t0 + 2 * TK);
      }
      __syncthreads();
    }

    // partial of this sequence piece: unnormalised o_lat (log2-domain max, sum)
    if (wave_live) {
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (h < H) {
        const int slot = blk + b;
        float *po = a.part_o + ((int64_t)slot * H + h) * R;
#pragma unroll
        for (int d = 0; d < NCT; ++d) {
          const int c = d * 16 + q * 4;
          if (c + 4 <= R) *reinterpret_cast<f32x4 *>(po + c) = o[d];
        }
        if (q == 0) {
          a.part_ml[((int64_t)slot * H + h) * 2 + 0] = m_run * sl2;
          a.part_ml[((int64_t)slot * H + h) * 2 + 1] = l_tot;
        }
      }
    }
    r0 = seg_end;
    ++b;
  }
#undef DEC_FETCH
#undef DEC_STASH
}

// Combine the pieces of sequence b: o_lat = sum_i w_i O_i / sum_i w_i l_i,
// w_i = exp2(m_i - max_i m_i).  A sequence with no valid rows gets NaN.
// One workgroup per (sequence, group of 8 heads).
constexpr int MERGE_HEADS = 8;

template <typename T, int R>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  __shared__ int sh[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    int before = 0, all = 0;
    for (int i = tid; i < a.B; i += 64) {
      const int n = seq_rows(a.lens, i, a.cap);
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
  const int n_b = seq_rows(a.lens, b, a.cap);
  const int h0 = blockIdx.y * MERGE_HEADS;
  if (n_b == 0) {
    for (int i = tid; i < MERGE_HEADS * R; i += 256) {
      const int h = h0 + i / R;
      if (h < a.H) reinterpret_cast<T *>(a.o_lat)[((int64_t)b * a.H + h) * R + i % R] = from_f32<T>(NAN);
    }
    return;
  }
  const int per = (total + a.n_blocks - 1) / a.n_blocks;
  const int i0 = start / per, i1 = (start + n_b - 1) / per;
  for (int hh = 0; hh < MERGE_HEADS; ++hh) {
    const int h = h0 + hh;
    if (h >= a.H) break;
    float M = -INFINITY;
    for (int i = i0; i <= i1; ++i) M = fmaxf(M, a.part_ml[((int64_t)(i + b) * a.H + h) * 2]);
    float L = 0.f;
    for (int i = i0; i <= i1; ++i) {
      const float *ml = a.part_ml + ((int64_t)(i + b) * a.H + h) * 2;
      L += exp2f(ml[0] - M) * ml[1];
    }
    const float invL = 1.0f / L;
    T *out = reinterpret_cast<T *>(a.o_lat) + ((int64_t)b * a.H + h) * R;
    for (int c = tid; c < R; c += 256) {
      float acc = 0.f;
      for (int i = i0; i <= i1; ++i) {
        const float w = exp2f(a.part_ml[((int64_t)(i + b) * a.H + h) * 2] - M);
        acc += w * a.part_o[((int64_t)(i + b) * a.H + h) * R + c];
      }
      out[c] = from_f32<T>(acc * invL);
    }
  }
}

template <typename T, int R, int DR>
hipError_t launch_t(const DecodeAttnArgs &a, hipStream_t st) {
  dim3 grid(a.n_blocks * ((a.H + HPB - 1) / HPB));
  size_t shm = (size_t)(a.B + 1) * sizeof(int);
  hipLaunchKernelGGL((decode_attn_kernel<T, R, DR>), grid, dim3(256), shm, st, a);
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_merge_t(const DecodeAttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((decode_merge_kernel<T, R>), dim3(a.B, (a.H + MERGE_HEADS - 1) / MERGE_HEADS),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int decode_blocks() { return 128; }

hipError_t launch_decode_attention(int dtype, int r, int dr, const DecodeAttnArgs &a,
                                   hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
#define MLA_DEC_CASE(R_, DR_)                                                        \
  if (r == R_ && dr == DR_)                                                          \
    return dtype == BF16 ? launch_t<bf16, R_, DR_>(a, st) : launch_t<float, R_, DR_>(a, st);
  MLA_DEC_CASE(16, 8)
  MLA_DEC_CASE(128, 32)
  MLA_DEC_CASE(512, 64)
#undef MLA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(int dtype, int r, const DecodeAttnArgs &a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
#define MLA_MERGE_CASE(R_)                                                           \
  if (r == R_) return dtype == BF16 ? launch_merge_t<bf16, R_>(a, st) : launch_merge_t<float, R_>(a, st);
  MLA_MERGE_CASE(16)
  MLA_MERGE_CASE(128)
  MLA_MERGE_CASE(512)
#undef MLA_MERGE_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
