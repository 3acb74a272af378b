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
// included) are laid end to end and cut into n_blocks equal ranges, one per
// workgroup, so long and short sequences load the GPU evenly.  A range that
// spans sequence boundaries yields one partial (unnormalised o_lat, running
// max, running sum) per sequence piece, in slot (block + b) -- unique because
// block and sequence indices both rise along the flattened rows.  A merge
// kernel combines the pieces of each sequence with log-sum-exp weights.
//
// Inside a workgroup: four waves, 32 heads each.  A wave computes S^T = C Q^T
// on 32x32 MFMA tiles (32 cache rows x 32 heads, K = 576), keeps the softmax
// online per head (each lane holds one head), and accumulates O^T += C^T P^T
// with P^T taken from the score accumulators in place.  Cache tiles are staged
// in LDS twice: row-major for the score product and transposed (latent part
// only) for the value product.

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int TK = 32;  // cache rows per tile
constexpr float LOG2E = 1.4426950408889634f;

template <typename T, int R, int DR>
struct DecCfg {
  using MF = Mfma32<T>;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int W = R + DR;
  static constexpr int WP = (W + MF::KSTEP - 1) / MF::KSTEP * MF::KSTEP;
  static constexpr int RP = (R + 31) / 32 * 32;
  static constexpr int CPITCH = WP + VEC;
  static constexpr int TPITCH = TK + VEC;
  static constexpr int NQF = WP / MF::KSTEP;
  static constexpr int NCT = RP / 32;
};

// Rows of sequence b in the flattened order: lens[b] + 1 for a valid length.
__device__ inline int seq_rows(const int32_t *lens, int b, int64_t cap) {
  const int32_t L = lens[b];
  return (L >= 0 && (int64_t)L < cap) ? L + 1 : 0;
}

template <typename T, int R, int DR>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  using C = DecCfg<T, R, DR>;
  using MF = typename C::MF;
  constexpr int VEC = C::VEC, W = C::W, WP = C::WP, RP = C::RP, CPITCH = C::CPITCH,
                TPITCH = C::TPITCH, NQF = C::NQF, NCT = C::NCT;
  __shared__ __attribute__((aligned(16))) T Cs[TK * CPITCH];
  __shared__ __attribute__((aligned(16))) T Ct[RP * TPITCH];
  extern __shared__ int starts[];  // [B + 1]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int B = a.B, H = a.H;
  const int blk = blockIdx.x;
  const int h = blockIdx.y * 128 + wave * 32 + l32;
  const bool wave_live = blockIdx.y * 128 + wave * 32 < H;

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

  if constexpr (RP > R) {
    for (int i = tid; i < (RP - R) * TPITCH; i += 256) Ct[R * TPITCH + i] = from_f32<T>(0.f);
  }
  const float sl2 = a.scale * LOG2E;
  const T *cache = reinterpret_cast<const T *>(a.cache);

  while (r0 < r1) {
    const int seg_end = min(r1, starts[b + 1]);
    const int t_begin = r0 - starts[b], t_end = seg_end - starts[b];
    const T *cb = cache + (int64_t)b * a.cap * W;

    typename MF::frag qf[NQF];
    const T *qp = reinterpret_cast<const T *>(a.q_lat) + ((int64_t)b * H + h) * W;
#pragma unroll
    for (int f = 0; f < NQF; ++f) {
      const int c = f * MF::KSTEP + g * MF::KPL;
      if constexpr (MF::KPL == 1) {
        qf[f] = (h < H && c < W) ? to_f32(qp[c]) : 0.f;
      } else {
        if (h < H && c < W) {
          uint4 v = *reinterpret_cast<const uint4 *>(qp + c);
          qf[f] = *reinterpret_cast<typename MF::frag *>(&v);
        } else {
          for (int e = 0; e < MF::KPL; ++e) qf[f][e] = from_f32<T>(0.f);
        }
      }
    }
    f32x16 o[NCT];
#pragma unroll
    for (int d = 0; d < NCT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int t0 = t_begin; t0 < t_end; t0 += TK) {
      __syncthreads();
      constexpr int CPR = WP / VEC;
      for (int c = tid; c < TK * CPR; c += 256) {
        const int jr = c / CPR, cc = (c - jr * CPR) * VEC;
        const int t = t0 + jr;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < t_end && cc < W) v = *reinterpret_cast<const uint4 *>(cb + (int64_t)t * W + cc);
        *reinterpret_cast<uint4 *>(&Cs[jr * CPITCH + cc]) = v;
        if (cc < R) {
          const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
          for (int i = 0; i < VEC; ++i) Ct[(cc + i) * TPITCH + jr] = e[i];
        }
      }
      __syncthreads();
      if (!wave_live) continue;

      f32x16 st;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        const typename MF::frag kf = *reinterpret_cast<const typename MF::frag *>(
            &Cs[l32 * CPITCH + f * MF::KSTEP + g * MF::KPL]);
        st = MF::mma(kf, qf[f], st);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = st[r] * sl2;
        if (t0 + acc_row(r, lane) >= t_end) s = -INFINITY;
        st[r] = s;
        mx = fmaxf(mx, s);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2f(st[r] - m_use);
        st[r] = pr;
        psum += pr;
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int d = 0; d < NCT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
#pragma unroll
      for (int u = 0; u < 16 / MF::KPL; ++u) {
        typename MF::frag pf;
        if constexpr (MF::KPL == 1) {
          pf = st[u];
        } else {
#pragma unroll
          for (int e = 0; e < MF::KPL; ++e) pf[e] = from_f32<T>(st[u * MF::KPL + e]);
        }
#pragma unroll
        for (int d = 0; d < NCT; ++d) {
          const T *row = &Ct[(d * 32 + l32) * TPITCH];
          typename MF::frag vf;
          if constexpr (MF::KPL == 1) {
            vf = to_f32(row[acc_row(u, lane)]);
          } else {
            const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + u * 16 + g * 4);
            const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + u * 16 + 8 + g * 4);
            vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          o[d] = MF::mma(vf, pf, o[d]);
        }
      }
    }

    // partial of this sequence piece: unnormalised o_lat, max (log2 domain), sum
    if (wave_live && h < H) {
      const int slot = blk + b;
      float *po = a.part_o + ((int64_t)slot * H + h) * R;
#pragma unroll
      for (int d = 0; d < NCT; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = d * 32 + acc_row(r, lane);
          if (c < R) po[c] = o[d][r];
        }
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      if (g == 0) {
        a.part_ml[((int64_t)slot * H + h) * 2 + 0] = m_run;
        a.part_ml[((int64_t)slot * H + h) * 2 + 1] = l_tot;
      }
    }
    r0 = seg_end;
    ++b;
  }
}

// Combine the pieces of sequence b: o_lat = sum_i w_i O_i / sum_i w_i l_i,
// w_i = exp2(m_i - max_i m_i).  A sequence with no valid rows gets NaN.
template <typename T, int R>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeAttnArgs a) {
  __shared__ int red[256];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  int before = 0, all = 0;
  for (int i = tid; i < a.B; i += 256) {
    const int n = seq_rows(a.lens, i, a.cap);
    all += n;
    if (i < b) before += n;
  }
  red[tid] = before;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const int start = red[0];
  __syncthreads();
  red[tid] = all;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const int total = red[0];
  const int n_b = seq_rows(a.lens, b, a.cap);
  T *out = reinterpret_cast<T *>(a.o_lat) + ((int64_t)b * a.H + h) * R;
  if (n_b == 0) {
    for (int c = tid; c < R; c += 256) out[c] = from_f32<T>(NAN);
    return;
  }
  const int per = (total + a.n_blocks - 1) / a.n_blocks;
  const int i0 = start / per, i1 = (start + n_b - 1) / per;
  float M = -INFINITY;
  for (int i = i0; i <= i1; ++i) M = fmaxf(M, a.part_ml[((int64_t)(i + b) * a.H + h) * 2]);
  float L = 0.f;
  for (int i = i0; i <= i1; ++i) {
    const float *ml = a.part_ml + ((int64_t)(i + b) * a.H + h) * 2;
    L += exp2f(ml[0] - M) * ml[1];
  }
  const float invL = 1.0f / L;
  for (int c = tid; c < R; c += 256) {
    float acc = 0.f;
    for (int i = i0; i <= i1; ++i) {
      const float w = exp2f(a.part_ml[((int64_t)(i + b) * a.H + h) * 2] - M);
      acc += w * a.part_o[((int64_t)(i + b) * a.H + h) * R + c];
    }
    out[c] = from_f32<T>(acc * invL);
  }
}

template <typename T, int R, int DR>
hipError_t launch_t(const DecodeAttnArgs &a, hipStream_t st) {
  dim3 grid(a.n_blocks, (a.H + 127) / 128);
  size_t shm = (size_t)(a.B + 1) * sizeof(int);
  hipLaunchKernelGGL((decode_attn_kernel<T, R, DR>), grid, dim3(256), shm, st, a);
  return hipGetLastError();
}

template <typename T, int R>
hipError_t launch_merge_t(const DecodeAttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((decode_merge_kernel<T, R>), dim3(a.B, a.H), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int decode_blocks() { return 256; }

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
