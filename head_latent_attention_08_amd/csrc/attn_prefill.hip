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
// operand; V is stored transposed in LDS so the matching A operand is two
// 8-byte LDS reads.  Query tiles are issued longest-first (causal work grows
// with the query index).

#include "common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int BQ = 128, BKV = 64;
constexpr float LOG2E = 1.4426950408889634f;

template <typename T, int DN, int DR, int DV>
struct AttnCfg {
  using MF = Mfma32<T>;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int DQK = DN + DR;
  static constexpr int DQKP = (DQK + MF::KSTEP - 1) / MF::KSTEP * MF::KSTEP;
  static constexpr int DVP = (DV + 31) / 32 * 32;
  static constexpr int KPITCH = DQKP + VEC;
  static constexpr int VPITCH = BKV + VEC;
  static constexpr int NQF = DQKP / MF::KSTEP;
  static constexpr int NDT = DVP / 32;
};

template <typename T>
__device__ inline uint4 ld16(const T *p) { return *reinterpret_cast<const uint4 *>(p); }

template <typename T, int DN, int DR, int DV>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs a) {
  using C = AttnCfg<T, DN, DR, DV>;
  using MF = typename C::MF;
  constexpr int VEC = C::VEC, DQK = C::DQK, DQKP = C::DQKP, KPITCH = C::KPITCH,
                VPITCH = C::VPITCH, NQF = C::NQF, NDT = C::NDT, DVP = C::DVP;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * KPITCH];
  __shared__ __attribute__((aligned(16))) T Vt[DVP * VPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int S = a.S, H = a.H;
  const int nq = (S + BQ - 1) / BQ;
  const int qt = nq - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int q0 = qt * BQ;
  const int qw0 = q0 + wave * 32;
  const int iq = qw0 + l32;  // this lane's query

  const int64_t bh = (int64_t)b * H + h;
  const T *qp = reinterpret_cast<const T *>(a.q) + bh * S * DQK;
  const T *kn = reinterpret_cast<const T *>(a.k_nope) + bh * S * DN;
  const T *kpe = reinterpret_cast<const T *>(a.k_pe) + (int64_t)b * S * a.ld_kpe;
  const T *vp = reinterpret_cast<const T *>(a.v) + bh * S * DV;

  // zero the padding rows of V^T once (d >= DV never gets written)
  if constexpr (DVP > DV) {
    for (int i = tid; i < (DVP - DV) * VPITCH; i += 256) Vt[DV * VPITCH + i] = from_f32<T>(0.f);
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
        for (int e = 0; e < MF::KPL; ++e) qf[f][e] = from_f32<T>(0.f);
      }
    }
  }

  f32x16 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * LOG2E;

  const int kv_end = min(S, q0 + BQ);
  for (int j0 = 0; j0 < kv_end; j0 += BKV) {
    __syncthreads();  // previous tile fully consumed
    // stage K = [k_nope ‖ k_pe] rows j0..j0+63 (zero outside) into LDS
    constexpr int CPR = DQKP / VEC;
    for (int c = tid; c < BKV * CPR; c += 256) {
      const int jr = c / CPR, cc = (c - jr * CPR) * VEC;
      const int j = j0 + jr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < S) {
        if (cc < DN) v = ld16(kn + (int64_t)j * DN + cc);
        else if (cc < DQK) v = ld16(kpe + (int64_t)j * a.ld_kpe + (cc - DN));
      }
      *reinterpret_cast<uint4 *>(&Ks[jr * KPITCH + cc]) = v;
    }
    // stage V^T: lane-consecutive keys so the 2-byte LDS writes do not collide
    constexpr int VCH = DV / VEC;
    for (int c = tid; c < BKV * VCH; c += 256) {
      const int jr = c & (BKV - 1), dc = c / BKV;
      const int j = j0 + jr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < S) v = ld16(vp + (int64_t)j * DV + dc * VEC);
      const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
      for (int i = 0; i < VEC; ++i) Vt[(dc * VEC + i) * VPITCH + jr] = e[i];
    }
    __syncthreads();

    if (j0 > qw0 + 31) continue;  // every key of the tile is after this wave's queries

    f32x16 st[BKV / 32];
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[jt][r] = 0.f;
#pragma unroll
      for (int f = 0; f < NQF; ++f) {
        const typename MF::frag kf = *reinterpret_cast<const typename MF::frag *>(
            &Ks[(jt * 32 + l32) * KPITCH + f * MF::KSTEP + g * MF::KPL]);
        st[jt] = MF::mma(kf, qf[f], st[jt]);
      }
    }
    // scale, causal mask, tile max of this lane's query
    const bool diag = j0 + BKV - 1 > qw0;
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = st[jt][r] * sl2;
        if (diag) {
          const int j = j0 + jt * 32 + acc_row(r, lane);
          if (j > iq) s = -INFINITY;
        }
        st[jt][r] = s;
        mx = fmaxf(mx, s);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2f(st[jt][r] - m_use);
        st[jt][r] = pr;
        psum += pr;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

    // O^T += V^T P^T, P^T taken from the score accumulators in place
#pragma unroll
    for (int jt = 0; jt < BKV / 32; ++jt) {
#pragma unroll
      for (int u = 0; u < 16 / MF::KPL; ++u) {
        typename MF::frag pf;
        if constexpr (MF::KPL == 1) {
          pf = st[jt][u];
        } else {
#pragma unroll
          for (int e = 0; e < MF::KPL; ++e) pf[e] = from_f32<T>(st[jt][u * MF::KPL + e]);
        }
#pragma unroll
        for (int d = 0; d < NDT; ++d) {
          const T *row = &Vt[(d * 32 + l32) * VPITCH + jt * 32];
          typename MF::frag vf;
          if constexpr (MF::KPL == 1) {
            vf = to_f32(row[acc_row(u, lane)]);
          } else {
            // k slots e = 0..7 hold keys (e/4)*8 + g*4 + e%4 of this 16-key slice
            const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + u * 16 + g * 4);
            const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + u * 16 + 8 + g * 4);
            vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          o[d] = MF::mma(vf, pf, o[d]);
        }
      }
    }
  }

  // normalise and store o[b, i, h, d]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (iq < S) {
    T *op = reinterpret_cast<T *>(a.o) + ((int64_t)b * S + iq) * (int64_t)H * DV + (int64_t)h * DV;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = d * 32 + acc_row(r, lane);
        if (dd < DV) op[dd] = from_f32<T>(o[d][r] * inv);
      }
  }
}

template <typename T, int DN, int DR, int DV>
hipError_t launch_t(const PrefillAttnArgs &a, hipStream_t st) {
  dim3 grid((a.S + BQ - 1) / BQ, a.H, a.B);
  hipLaunchKernelGGL((prefill_attn_kernel<T, DN, DR, DV>), grid, dim3(256), 0, st, a);
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
