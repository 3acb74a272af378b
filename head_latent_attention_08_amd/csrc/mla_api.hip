// C ABI of the MLA forward: argument checks, workspace carving, launch
// sequences for prefill and absorbed decode, and the standalone RoPE.
//
// The prefill follows MultiHeadLatentAttention.forward of "The Evolving
// Transformer -- DeepSeek V2 & V3" (section 01) step by step:
//   1. down projections  [c_q ‖ c_kv ‖ k_pe] = x [w_down_q; w_down_kv; w_kr]^T
//   2. RMSNorm of c_q      3. RoPE of k_pe (shared key)
//   4. q up-projection into head-major q = [q_nope ‖ q_pe], then RoPE of q_pe
//   5. kv up-projection into head-major k_nope and v
//   6. causal attention  7. output projection y = o wo^T
// The decode step replaces 5-6 by the absorbed form over the latent cache.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/mla.h"
#include "internal.h"

using namespace mla;

namespace {

thread_local std::string g_err;
thread_local void *const *g_events = nullptr;
thread_local int g_n_events = 0;

mla_status fail(mla_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status fail(mla_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

mla_status hip_fail(hipError_t e, const char *where) {
  return fail(MLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define MLA_HIP(call, where)                         \
  do {                                               \
    hipError_t e_ = (call);                          \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

// Record stage event k on the stream when the caller asked for stage timing.
hipError_t mark(int k, hipStream_t st) {
  if (g_events && k < g_n_events && g_events[k])
    return hipEventRecord((hipEvent_t)g_events[k], st);
  return hipSuccess;
}

#define MLA_MARK(k) MLA_HIP(mark((k), st), "stage event")

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

mla_status check_rope(const mla_rope_params *rp, int rope_dim) {
  if (!rp) return fail(MLA_ERR_INVALID_ARGUMENT, "rope params are NULL");
  if (rp->convention != MLA_ROPE_HALF_SPLIT && rp->convention != MLA_ROPE_INTERLEAVED)
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope convention %d is neither 0 nor 1",
                rp->convention);
  if (!(rp->theta > 1.0f) || !std::isfinite(rp->theta))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope theta must be finite and > 1");
  if (!(rp->factor >= 1.0f) || !std::isfinite(rp->factor))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope factor must be finite and >= 1");
  if (rp->factor > 1.0f) {
    if (rp->original_max_position < 1)
      return fail(MLA_ERR_INVALID_ARGUMENT, "YaRN needs original_max_position >= 1");
    if (!(rp->beta_fast > 0) || !(rp->beta_slow > 0))
      return fail(MLA_ERR_INVALID_ARGUMENT, "YaRN betas must be > 0");
  }
  if (rope_dim < 2 || rope_dim > 128 || (rope_dim & 1))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rope_dim %d must be even and in [2, 128]", rope_dim);
  return MLA_OK;
}

double yarn_mscale(double s, double m) { return s <= 1.0 ? 1.0 : 0.1 * m * std::log(s) + 1.0; }

// Frequencies of pair i: theta^(-2i/d).  With YaRN (factor > 1) the pairs
// between the correction indices of beta_fast and beta_slow blend linearly
// (in pair index) from the original frequency to frequency / factor; pairs
// past the slow bound are fully divided.  The cos/sin amplitude is
// mscale(factor, mscale) / mscale(factor, mscale_all_dim).
RopeTab make_rope_tab(const mla_rope_params &rp, int rope_dim) {
  RopeTab t;
  std::memset(&t, 0, sizeof t);
  const int P = rope_dim / 2;
  t.pairs = P;
  t.convention = rp.convention;
  const double theta = rp.theta;
  for (int i = 0; i < P; ++i) t.inv_freq[i] = std::pow(theta, -2.0 * i / rope_dim);
  t.amp = 1.0f;
  if (rp.factor > 1.0f) {
    const double f = rp.factor;
    auto corr = [&](double rot) {
      return rope_dim * std::log(rp.original_max_position / (rot * 2.0 * M_PI)) /
             (2.0 * std::log(theta));
    };
    double lo = std::floor(corr(rp.beta_fast));
    double hi = std::ceil(corr(rp.beta_slow));
    if (lo < 0) lo = 0;
    if (hi > rope_dim - 1) hi = rope_dim - 1;
    if (hi == lo) hi += 0.001;
    for (int i = 0; i < P; ++i) {
      double ramp = (i - lo) / (hi - lo);
      ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
      t.inv_freq[i] = t.inv_freq[i] * (1.0 - ramp) + t.inv_freq[i] / f * ramp;
    }
    t.amp = (float)(yarn_mscale(f, rp.mscale) / yarn_mscale(f, rp.mscale_all_dim));
  }
  return t;
}

float resolve_scale(const mla_config &c) {
  if (c.softmax_scale > 0) return c.softmax_scale;
  double s = 1.0 / std::sqrt((double)(c.qk_nope_head_dim + c.qk_rope_head_dim));
  if (c.rope.factor > 1.0f) {
    double m = yarn_mscale(c.rope.factor, c.rope.mscale_all_dim);
    s *= m * m;
  }
  return (float)s;
}

bool prefill_instance(const mla_config &c) {
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim;
  return (dn == 16 && dr == 8 && dv == 16) || (dn == 64 && dr == 32 && dv == 64) ||
         (dn == 128 && dr == 64 && dv == 128);
}

bool decode_instance(const mla_config &c) {
  const int r = c.kv_lora_rank, dr = c.qk_rope_head_dim;
  return (r == 16 && dr == 8) || (r == 128 && dr == 32) ||
         (r == 512 && dr == 64 && c.dtype == MLA_DTYPE_BF16);
}

mla_status check_config(const mla_config *c) {
  if (!c) return fail(MLA_ERR_INVALID_ARGUMENT, "config is NULL");
  const struct {
    const char *name;
    int v;
  } dims[] = {{"hidden_size", c->hidden_size},           {"num_heads", c->num_heads},
              {"q_lora_rank", c->q_lora_rank},           {"kv_lora_rank", c->kv_lora_rank},
              {"qk_nope_head_dim", c->qk_nope_head_dim}, {"qk_rope_head_dim", c->qk_rope_head_dim},
              {"v_head_dim", c->v_head_dim}};
  for (auto &d : dims) {
    if (d.v < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "%s = %d must be >= 1", d.name, d.v);
    if (d.name != std::string("num_heads") && d.v % 8)
      return fail(MLA_ERR_INVALID_ARGUMENT, "%s = %d must be a multiple of 8", d.name, d.v);
  }
  if (c->num_heads > 65535) return fail(MLA_ERR_INVALID_ARGUMENT, "num_heads too large");
  if (c->dtype != MLA_DTYPE_F32 && c->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dtype %d is neither 0 (fp32) nor 1 (bf16)", c->dtype);
  if (!(c->rms_norm_eps >= 0.0f) || !std::isfinite(c->rms_norm_eps))
    return fail(MLA_ERR_INVALID_ARGUMENT, "rms_norm_eps must be finite and >= 0");
  if (!std::isfinite(c->softmax_scale))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  return check_rope(&c->rope, c->qk_rope_head_dim);
}

mla_status check_weights(const mla_weights *w) {
  if (!w) return fail(MLA_ERR_INVALID_ARGUMENT, "weights are NULL");
  const struct {
    const char *name;
    const void *p;
  } ws[] = {{"w_down_q", w->w_down_q},   {"q_norm", w->q_norm}, {"w_up_q", w->w_up_q},
            {"w_qr", w->w_qr},           {"w_down_kv", w->w_down_kv}, {"w_kr", w->w_kr},
            {"w_up_k", w->w_up_k},       {"w_up_v", w->w_up_v}, {"wo", w->wo}};
  for (auto &x : ws) {
    if (!x.p) return fail(MLA_ERR_INVALID_ARGUMENT, "weight %s is NULL", x.name);
    if (!aligned16(x.p))
      return fail(MLA_ERR_INVALID_ARGUMENT, "weight %s is not 16-byte aligned", x.name);
  }
  if (w->kv_norm && !aligned16(w->kv_norm))  // optional: NULL means no norm on c_kv
    return fail(MLA_ERR_INVALID_ARGUMENT, "weight kv_norm is not 16-byte aligned");
  return MLA_OK;
}

// RMSNorm of c_q (always) and of c_kv (when kv_norm gains are given) in the
// down-projection output rows [c_q ‖ c_kv ‖ k_pe] of pitch ld.
hipError_t launch_down_norms(const mla_config &c, const mla_weights *w, char *down, int64_t rows,
                             int64_t ld, hipStream_t st) {
  hipError_t e = launch_rmsnorm(c.dtype, down, rows, ld, c.q_lora_rank, w->q_norm, c.rms_norm_eps, st);
  if (e != hipSuccess || !w->kv_norm) return e;
  return launch_rmsnorm(c.dtype, down + (size_t)c.q_lora_rank * dtype_size(c.dtype), rows, ld,
                        c.kv_lora_rank, w->kv_norm, c.rms_norm_eps, st);
}

struct PrefillPlan {
  int64_t ld_down;
  size_t off_down, off_q, off_kn, off_v, off_o, total;
  size_t off_qrms;  // split RMSNorm of c_q: [B*S, r_q / 64] fp32 partial sums of squares
  bool q_norm_split;
  size_t off_rope;  // q_pe rotated in the q up-projection: [B*S, d_r] fp32 cos | sin per token
  bool q_rope_fused;
  size_t off_start, off_last, off_pos, off_valid, off_ok;  // key-range prefills only
};

// The prefill's fused down-projection [c_q ‖ c_kv ‖ k_pe] = x [w_down_q;
// w_down_kv; w_kr]^T and its q up-projection [q_nope ‖ q_pe] per head =
// c_qn [w_up_q; w_qr]^T (w, x and the outputs may be NULL where only the
// shapes matter).
GemmDesc down_proj_desc(const mla_config &c, int64_t M, const mla_weights *w, const void *x, void *down,
                        int64_t ld_down) {
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank, dr = c.qk_rope_head_dim;
  GemmDesc g;
  g.dtype = c.dtype;
  g.M = (int)M;
  g.N = rq + rkv + dr;
  g.K = D;
  g.A = x;
  g.lda = D;
  g.S = (int)M;
  g.H = 1;
  g.nseg = 3;
  g.seg[0] = GemmSeg{w ? w->w_down_q : nullptr, D, 0, down, rq, ld_down, 0};
  g.seg[1] = GemmSeg{w ? w->w_down_kv : nullptr, D, rq, down, rkv, ld_down, rq};
  g.seg[2] = GemmSeg{w ? w->w_kr : nullptr, D, rq + rkv, down, dr, ld_down, rq + rkv};
  return g;
}

GemmDesc q_up_desc(const mla_config &c, int64_t M, int64_t S, const mla_weights *w, const void *down,
                   int64_t ld_down, void *q) {
  const int H = c.num_heads, rq = c.q_lora_rank, dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim;
  const int dqk = dn + dr;
  GemmDesc g;
  g.dtype = c.dtype;
  g.M = (int)M;
  g.N = H * dqk;
  g.K = rq;
  g.A = down;
  g.lda = ld_down;
  g.S = (int)S;
  g.H = H;
  g.nseg = 2;
  g.seg[0] = GemmSeg{w ? w->w_up_q : nullptr, rq, 0, q, dn, dqk, 0};
  g.seg[1] = GemmSeg{w ? w->w_qr : nullptr, rq, H * dn, q, dr, dqk, dn};
  return g;
}

PrefillPlan plan_prefill(const mla_config &c, int64_t B, int64_t S, bool varlen = false) {
  const size_t es = dtype_size(c.dtype);
  const int64_t M = B * S, H = c.num_heads;
  PrefillPlan p;
  p.ld_down = (int64_t)round_up(c.q_lora_rank + c.kv_lora_rank + c.qk_rope_head_dim, 8);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  p.off_down = take((size_t)M * p.ld_down * es);
  p.off_q = take((size_t)M * H * (c.qk_nope_head_dim + c.qk_rope_head_dim) * es);
  p.off_kn = take((size_t)M * H * c.qk_nope_head_dim * es);
  p.off_v = take((size_t)M * H * c.v_head_dim * es);
  p.off_o = take((size_t)M * H * c.v_head_dim * es);
  p.off_start = p.off_last = p.off_pos = p.off_valid = p.off_ok = 0;
  if (varlen) {
    p.off_start = take((size_t)M * sizeof(int32_t));
    p.off_last = take((size_t)M * sizeof(int32_t));
    p.off_pos = take((size_t)M * sizeof(int32_t));
    p.off_valid = take((size_t)M * sizeof(int32_t));
    p.off_ok = take(sizeof(int32_t));
  }
  // RMSNorm(c_q) split over the two products' epilogues when both run on the
  // large-tile kernel (bf16): the down-projection leaves per-row partial sums
  // of squares of c_q (per 64 columns) and stores c_q times the gains, the q
  // up-projection scales each output row by the row's 1 / rms
  p.q_norm_split = c.dtype == MLA_DTYPE_BF16 && c.q_lora_rank % 64 == 0 &&
                   gemm_uses_large_tiles(down_proj_desc(c, M, nullptr, nullptr, nullptr, p.ld_down)) &&
                   gemm_uses_large_tiles(q_up_desc(c, M, S, nullptr, nullptr, p.ld_down, nullptr));
  p.off_qrms = take(p.q_norm_split ? (size_t)M * (c.q_lora_rank / 64) * sizeof(float) : 0);
  // RoPE of q_pe in the q up-projection's epilogue where its tiles hold whole
  // q_pe heads: the k_pe rotation (which runs first, at the same tokens'
  // positions) leaves every token's cos / sin in a table for it
  p.q_rope_fused = c.dtype == MLA_DTYPE_BF16 &&
                   gemm_rope_fusable(q_up_desc(c, M, S, nullptr, nullptr, p.ld_down, nullptr), 1);
  p.off_rope = take(p.q_rope_fused ? (size_t)M * c.qk_rope_head_dim * sizeof(float) : 0);
  p.total = off;
  return p;
}

struct DecodePlan {
  int64_t ld_down;
  int n_blocks;
  size_t off_down, off_qn, off_qlat, off_po, off_pml, off_olat, off_o, off_gemm, gemm_bytes,
      off_pos, total;
};

// Workspace of a decode step of B sequences with T new tokens each: the
// per-token buffers hold B*T rows; the attention partials cover T*H query
// heads (token t's head h is query head t*H + h).
DecodePlan plan_decode(const mla_config &c, int64_t Bseq, int64_t T = 1) {
  const int64_t B = Bseq * T;  // token rows
  const size_t es = dtype_size(c.dtype);
  const int64_t H = c.num_heads, r = c.kv_lora_rank, dr = c.qk_rope_head_dim;
  DecodePlan p;
  p.ld_down = (int64_t)round_up(c.q_lora_rank + r + dr, 8);
  p.n_blocks = decode_blocks((int)T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  p.off_down = take((size_t)B * p.ld_down * es);
  p.off_qn = take((size_t)B * H * c.qk_nope_head_dim * es);
  p.off_qlat = take((size_t)B * H * (r + dr) * es);
  // attention partials: blocks of 32 heads x (r rounded up to 32) channels,
  // bf16 for a bf16 cache, else fp32
  p.off_po = take((size_t)(p.n_blocks + Bseq) * ((T * H + 31) / 32) * 32 * ((r + 31) / 32 * 32) *
                  (es == 2 ? es : sizeof(float)));
  p.off_pml = take((size_t)(p.n_blocks + Bseq) * T * H * 2 * sizeof(float));
  p.off_olat = take((size_t)B * H * r * es);
  p.off_o = take((size_t)B * H * c.v_head_dim * es);
  // split-K partials of the weight-streaming projections (largest of the four)
  const int D = c.hidden_size, rq = c.q_lora_rank, dn = c.qk_nope_head_dim, dv = c.v_head_dim;
  size_t gb = gemm_scratch_bytes(c.dtype, (int)B, rq + (int)r + (int)dr, D, 1);
  gb = std::max(gb, gemm_scratch_bytes(c.dtype, (int)B, (int)H * (dn + (int)dr), rq, 1));
  gb = std::max(gb, gemm_scratch_bytes(c.dtype, (int)B, dv, (int)r, (int)H));
  gb = std::max(gb, gemm_scratch_bytes(c.dtype, (int)B, D, (int)H * dv, 1));
  p.gemm_bytes = gb;
  p.off_gemm = take(gb);
  p.off_pos = take((size_t)B * sizeof(int32_t));  // positions lens[b] + t (T > 1)
  p.total = off;
  return p;
}

mla_status check_prefill_sizes(const mla_config *cfg, int64_t B, int64_t S) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (B < 1 || S < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "batch and seq must be >= 1");
  if (B > 65535 || S > (1 << 24) || B * S > (1LL << 30))
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch %lld x seq %lld is too large", (long long)B,
                (long long)S);
  if (!prefill_instance(*cfg))
    return fail(MLA_ERR_UNSUPPORTED,
                "head dims (nope %d, rope %d, v %d) are not instantiated; supported: "
                "(16,8,16), (64,32,64), (128,64,128)",
                cfg->qk_nope_head_dim, cfg->qk_rope_head_dim, cfg->v_head_dim);
  return MLA_OK;
}

mla_status check_decode_sizes(const mla_config *cfg, int64_t B, int64_t cap, int64_t T = 1) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (B < 1 || B > 4096) return fail(MLA_ERR_INVALID_ARGUMENT, "batch must be in [1, 4096]");
  if (T < 1 || T > 256) return fail(MLA_ERR_INVALID_ARGUMENT, "q_len must be in [1, 256]");
  if (T > cap) return fail(MLA_ERR_INVALID_ARGUMENT, "q_len exceeds cache_capacity");
  if (cap < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "cache_capacity must be >= 1");
  if (B * cap > (1LL << 30))
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch x cache_capacity is too large");
  if (!decode_instance(*cfg))
    return fail(MLA_ERR_UNSUPPORTED,
                "(kv_lora_rank %d, rope %d) is not instantiated for this dtype; supported: "
                "(16,8), (128,32), and (512,64) in bf16",
                cfg->kv_lora_rank, cfg->qk_rope_head_dim);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char *mla_last_error(void) { return g_err.c_str(); }

mla_status mla_set_stage_events(void *const *events, int32_t n_events) {
  if (n_events < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_events must be >= 0");
  g_events = (n_events > 0) ? events : nullptr;
  g_n_events = g_events ? n_events : 0;
  return MLA_OK;
}

const char *mla_version(void) { return "mla-mi355x 0.1.0 (gfx950)"; }

float mla_softmax_scale(const mla_config *cfg) {
  if (!cfg) return 0.f;
  return resolve_scale(*cfg);
}

mla_status mla_prefill_workspace_size(const mla_config *cfg, int64_t batch, int64_t seq,
                                      size_t *bytes) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_prefill(*cfg, batch, seq).total;
  return MLA_OK;
}

mla_status mla_prefill_layout_of(const mla_config *cfg, int64_t batch, int64_t seq,
                                 mla_prefill_layout *layout) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if (!layout) return fail(MLA_ERR_INVALID_ARGUMENT, "layout is NULL");
  const PrefillPlan p = plan_prefill(*cfg, batch, seq);
  const size_t es = dtype_size(cfg->dtype);
  layout->c_q = p.off_down;
  layout->c_kv = p.off_down + (size_t)cfg->q_lora_rank * es;
  layout->k_pe = p.off_down + (size_t)(cfg->q_lora_rank + cfg->kv_lora_rank) * es;
  layout->q = p.off_q;
  layout->k_nope = p.off_kn;
  layout->v = p.off_v;
  layout->o = p.off_o;
  layout->ld_down = p.ld_down;
  layout->q_rms_part = p.off_qrms;
  layout->q_rms_chunks = p.q_norm_split ? cfg->q_lora_rank / 64 : 0;
  layout->total = p.total;
  return MLA_OK;
}

// The prefill of B equal-length sequences, or (cu_seqlens set) of n_seq
// packed sequences of different lengths run as one stream of seq tokens.
static mla_status prefill_common(const mla_config *cfg, const mla_weights *w, const void *x,
                                 int64_t batch, int64_t seq, void *y, void *latent_out,
                                 void *workspace, size_t workspace_bytes, void *hip_stream,
                                 const int32_t *cu_seqlens, int64_t n_seq) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!x || !y || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, y and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) ||
      (latent_out && !aligned16(latent_out)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, y, latent_out and workspace must be 16-byte aligned");
  const mla_config &c = *cfg;
  const bool varlen = cu_seqlens != nullptr;
  const PrefillPlan p = plan_prefill(c, batch, seq, varlen);
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, p.total);

  hipStream_t st = (hipStream_t)hip_stream;
  const size_t es = dtype_size(c.dtype);
  char *ws = (char *)workspace;
  char *down = ws + p.off_down;
  char *q = ws + p.off_q;
  char *kn = ws + p.off_kn;
  char *v = ws + p.off_v;
  char *o = ws + p.off_o;
  const int B = (int)batch, S = (int)seq, M = B * S, H = c.num_heads;
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim;
  const int dqk = dn + dr;
  const RopeTab tab = make_rope_tab(c.rope, dr);
  // packed sequences: per token its sequence start and position
  int32_t *vl_start = varlen ? reinterpret_cast<int32_t *>(ws + p.off_start) : nullptr;
  int32_t *vl_last = varlen ? reinterpret_cast<int32_t *>(ws + p.off_last) : nullptr;
  int32_t *vl_pos = varlen ? reinterpret_cast<int32_t *>(ws + p.off_pos) : nullptr;
  int32_t *vl_valid = varlen ? reinterpret_cast<int32_t *>(ws + p.off_valid) : nullptr;
  int32_t *vl_ok = varlen ? reinterpret_cast<int32_t *>(ws + p.off_ok) : nullptr;

  // 1. [c_q ‖ c_kv ‖ k_pe] = x [w_down_q; w_down_kv; w_kr]^T
  MLA_MARK(0);
  if (varlen)
    MLA_HIP(launch_varlen_index(cu_seqlens, (int)n_seq, M, vl_start, vl_last, vl_pos, vl_valid,
                                vl_ok, st),
            "sequence offsets");
  float *qrms = reinterpret_cast<float *>(ws + p.off_qrms);
  {
    GemmDesc g = down_proj_desc(c, M, w, x, down, p.ld_down);
    if (p.q_norm_split) {
      g.rn_part = qrms;
      g.rn_gain = w->q_norm;
      g.rn_cols = rq;
    }
    MLA_HIP(launch_gemm(g, st), "down projection");
  }
  // 2. RMSNorm(c_q) (here unless split over the projections' epilogues), and
  // of c_kv when kv_norm gains are given
  MLA_MARK(1);
  if (p.q_norm_split) {
    if (w->kv_norm)
      MLA_HIP(launch_rmsnorm(c.dtype, down + (size_t)rq * es, M, p.ld_down, rkv, w->kv_norm, c.rms_norm_eps, st),
              "rmsnorm c_kv");
  } else {
    MLA_HIP(launch_down_norms(c, w, down, M, p.ld_down, st), "rmsnorm");
  }
  // 3. RoPE of the shared key at positions 0..S-1
  MLA_MARK(2);
  float *rope_tab = p.q_rope_fused ? reinterpret_cast<float *>(ws + p.off_rope) : nullptr;
  MLA_HIP(launch_rope(c.dtype, down + (size_t)(rq + rkv) * es, M, S, (int64_t)S * p.ld_down,
                      p.ld_down, 1, 0, vl_pos, tab, st, rope_tab),
          "rope k_pe");
  if (latent_out)
    MLA_HIP(launch_copy_rows(c.dtype, latent_out, rkv + dr, down + (size_t)rq * es, p.ld_down, M,
                             rkv + dr, st),
            "latent copy");
  // 4. q = [q_nope ‖ q_pe] per head, then RoPE of q_pe
  MLA_MARK(3);
  {
    GemmDesc g = q_up_desc(c, M, S, w, down, p.ld_down, q);
    if (p.q_norm_split) {
      g.rs_part = qrms;
      g.rs_chunks = rq / 64;
      g.rs_eps = c.rms_norm_eps;
    }
    if (p.q_rope_fused) {
      g.rope_tab = rope_tab;
      g.rope_seg = 1;
      g.rope_conv = c.rope.convention;
    }
    MLA_HIP(launch_gemm(g, st), "q up-projection");
  }
  MLA_MARK(4);
  if (!p.q_rope_fused)
    MLA_HIP(launch_rope(c.dtype, q + (size_t)dn * es, M, S, (int64_t)H * S * dqk, dqk, H,
                        (int64_t)S * dqk, vl_pos, tab, st),
            "rope q_pe");
  // 5. k_nope [B, H, S, d_n] and v channel-major [B, H, d_v, S] per head
  MLA_MARK(5);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = M;
    g.N = H * (dn + dv);
    g.K = rkv;
    g.A = down + (size_t)rq * es;
    g.lda = p.ld_down;
    g.S = S;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_k, rkv, 0, kn, dn, dn, 0};
    g.seg[1] = GemmSeg{w->w_up_v, rkv, H * dn, v, dv, dv, 0, 1};  // v channel-major
    MLA_HIP(launch_gemm(g, st), "kv up-projection");
  }
  // 6. causal attention
  MLA_MARK(6);
  {
    PrefillAttnArgs a;
    a.q = q;
    a.k_nope = kn;
    a.k_pe = down + (size_t)(rq + rkv) * es;
    a.ld_kpe = p.ld_down;
    a.vt = v;
    a.o = o;
    a.B = B;
    a.S = S;
    a.H = H;
    a.scale = resolve_scale(c);
    a.kv_lo = vl_start;
    a.kv_hi = vl_last;
    a.valid = vl_valid;
    a.Sk = S;
    MLA_HIP(launch_prefill_attention(c.dtype, dn, dr, dv, a, st), "attention");
  }
  // 7. y = o wo^T
  MLA_MARK(7);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = M;
    g.N = D;
    g.K = H * dv;
    g.A = o;
    g.lda = (int64_t)H * dv;
    g.S = M;
    g.H = 1;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->wo, (int64_t)H * dv, 0, y, D, D, 0};
    MLA_HIP(launch_gemm(g, st), "output projection");
  }
  MLA_MARK(8);
  return MLA_OK;
}

mla_status mla_prefill_forward(const mla_config *cfg, const mla_weights *w, const void *x,
                               int64_t batch, int64_t seq, void *y, void *latent_out,
                               void *workspace, size_t workspace_bytes, void *hip_stream) {
  return prefill_common(cfg, w, x, batch, seq, y, latent_out, workspace, workspace_bytes,
                        hip_stream, nullptr, 0);
}

// ---------------------------------------------------------------- MLA backward
// Every gradient of y = MLA(x) for an upstream dy: the forward's steps are
// run again (the intermediates the backward reads land in the workspace),
// then the chain rule back through them, in reverse order.
namespace {

struct BackwardPlan {
  PrefillPlan fwd;
  size_t off_cq_raw, off_ckv_raw, off_vh, off_kh, off_oh, off_doh, off_dqh, off_dkh, off_dvh, off_att,
      off_pos, off_gq, off_gkv, off_dcqn, off_dckv, off_ddown, off_wq, off_wkv, off_wd, off_rms, off_tr, off_dwd, total;
};

// Elements of transposed operand copies a backward product C [M, N] =
// op(A) op(B) (contraction K) needs: bf16 products the large-tile kernel
// takes get their transposed operands (A stored [K][M], B stored [K][N])
// rewritten K-contiguous, an HBM-bound pass that the general kernel's
// strided reads of the same operands cost many times over.
size_t bwd_tr_elems(int dtype, int64_t M, int64_t N, int64_t K, bool a_km, bool b_kn) {
  if (!(a_km || b_kn) || M % 8 || N % 8 || !gemm_takes_large_tiles(dtype, (int)M, (int)N, (int)K)) return 0;
  return (a_km ? round_up((size_t)(M * K), 128) : 0) + (b_kn ? (size_t)(N * K) : 0);
}

BackwardPlan plan_backward(const mla_config &c, int64_t B, int64_t S) {
  BackwardPlan p;
  p.fwd = plan_prefill(c, B, S);
  const size_t es = dtype_size(c.dtype);
  const int64_t M = B * S, H = c.num_heads;
  const int64_t rq = c.q_lora_rank, rkv = c.kv_lora_rank, D = c.hidden_size;
  const int64_t dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim;
  size_t off = p.fwd.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  p.off_cq_raw = take((size_t)M * rq * es);
  p.off_ckv_raw = take((size_t)M * rkv * es);
  p.off_vh = take((size_t)M * H * dv * es);
  p.off_kh = take((size_t)M * H * (dn + dr) * es);
  p.off_oh = take((size_t)M * H * dv * es);
  p.off_doh = take((size_t)M * H * dv * es);
  p.off_dqh = take((size_t)M * H * (dn + dr) * es);
  p.off_dkh = take((size_t)M * H * (dn + dr) * es);
  p.off_dvh = take((size_t)M * H * dv * es);
  p.off_att = take((size_t)M * H * 2 * sizeof(float));
  p.off_pos = take((size_t)M * sizeof(int32_t));
  p.off_gq = take((size_t)M * H * (dn + dr) * es);
  p.off_gkv = take((size_t)M * H * (dn + dv) * es);
  p.off_dcqn = take((size_t)M * rq * es);
  p.off_dckv = take((size_t)M * rkv * es);
  p.off_ddown = take((size_t)M * p.fwd.ld_down * es);
  p.off_wq = take((size_t)H * (dn + dr) * rq * es);
  p.off_wkv = take((size_t)H * (dn + dv) * rkv * es);
  p.off_wd = take((size_t)(rq + rkv + dr) * D * es);
  p.off_rms = take(std::max(rmsnorm_backward_scratch_floats(M, (int)rq), rmsnorm_backward_scratch_floats(M, (int)rkv)) *
                   sizeof(float));
  // the largest transposed-operand need over the backward's products
  const int dt = c.dtype;
  const size_t tr = std::max({bwd_tr_elems(dt, D, H * dv, M, true, true), bwd_tr_elems(dt, M, H * dv, D, false, true),
                              bwd_tr_elems(dt, H * dn, rq, M, true, true), bwd_tr_elems(dt, H * dr, rq, M, true, true),
                              bwd_tr_elems(dt, M, rq, H * (dn + dr), false, true),
                              bwd_tr_elems(dt, H * dn, rkv, M, true, true), bwd_tr_elems(dt, H * dv, rkv, M, true, true),
                              bwd_tr_elems(dt, M, rkv, H * (dn + dv), false, true),
                              bwd_tr_elems(dt, M, D, rq + rkv + dr, false, true), bwd_tr_elems(dt, rq, D, M, true, true),
                              bwd_tr_elems(dt, rkv, D, M, true, true), bwd_tr_elems(dt, dr, D, M, true, true),
                              bwd_tr_elems(dt, rq + rkv + dr, D, M, true, true)});
  p.off_tr = take(tr * es);
  // the stacked down-projection weights' gradient [r_q + r_kv + d_r, D]
  p.off_dwd = take((size_t)(rq + rkv + dr) * D * es);
  p.total = off;
  return p;
}

// A plain row-major product C [M, N] (pitch ldc) = op(A) op(B): A stored
// [M][K] (pitch lda) or, a_km, [K][M]; B stored [N][K] or, b_kn, [K][N].
hipError_t plain_gemm(int dtype, const void *A, int64_t lda, bool a_km, const void *B, int64_t ldb, bool b_kn,
                      void *C, int64_t ldc, int M, int N, int K, hipStream_t st) {
  GemmDesc g;
  g.dtype = dtype;
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.a_km = a_km;
  g.b_kn = b_kn;
  g.S = M;
  g.H = 1;
  g.nseg = 1;
  g.seg[0] = GemmSeg{B, ldb, 0, C, N, ldc, 0};
  return launch_gemm(g, st);
}

// plain_gemm for the backward's products, with the transposed operands of
// those bwd_tr_elems names rewritten K-contiguous into tr first.
hipError_t bwd_gemm(int dtype, const void *A, int64_t lda, bool a_km, const void *B, int64_t ldb, bool b_kn, void *C,
                    int64_t ldc, int M, int N, int K, char *tr, hipStream_t st) {
  if (bwd_tr_elems(dtype, M, N, K, a_km, b_kn) > 0) {
    char *t = tr;
    if (a_km) {
      hipError_t e = launch_transpose(A, lda, K, M, t, K, st);
      if (e != hipSuccess) return e;
      A = t;
      lda = K;
      t += round_up((size_t)M * K, 128) * 2;  // bf16
    }
    if (b_kn) {
      hipError_t e = launch_transpose(B, ldb, K, N, t, K, st);
      if (e != hipSuccess) return e;
      B = t;
      ldb = K;
    }
    a_km = b_kn = false;
  }
  return plain_gemm(dtype, A, lda, a_km, B, ldb, b_kn, C, ldc, M, N, K, st);
}

}  // namespace

mla_status mla_backward_workspace_size(const mla_config *cfg, int64_t batch, int64_t seq, size_t *bytes) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (batch * seq * cfg->num_heads > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch x seq x num_heads must stay below 2^31");
  *bytes = plan_backward(*cfg, batch, seq).total;
  return MLA_OK;
}

mla_status mla_backward(const mla_config *cfg, const mla_weights *w, const void *x, int64_t batch, int64_t seq,
                        const void *dy, void *dx, const mla_weight_grads *grads, void *workspace,
                        size_t workspace_bytes, void *hip_stream) {
  size_t need = 0;
  mla_status s = mla_backward_workspace_size(cfg, batch, seq, &need);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!x || !dy || !dx || !workspace || !grads)
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, dy, dx, grads and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(workspace))
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, dy, dx and workspace must be 16-byte aligned");
  {
    const struct {
      const char *name;
      const void *p;
    } gs[] = {{"w_down_q", grads->w_down_q}, {"q_norm", grads->q_norm}, {"w_up_q", grads->w_up_q},
              {"w_qr", grads->w_qr},         {"w_down_kv", grads->w_down_kv}, {"w_kr", grads->w_kr},
              {"w_up_k", grads->w_up_k},     {"w_up_v", grads->w_up_v},       {"wo", grads->wo}};
    for (auto &g : gs)
      if (!g.p || !aligned16(g.p)) return fail(MLA_ERR_INVALID_ARGUMENT, "gradient %s is NULL or not 16-byte aligned", g.name);
    if (w->kv_norm && (!grads->kv_norm || !aligned16(grads->kv_norm)))
      return fail(MLA_ERR_INVALID_ARGUMENT, "gradient kv_norm is NULL or not 16-byte aligned (weights carry kv_norm)");
  }
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);

  const mla_config &c = *cfg;
  const BackwardPlan p = plan_backward(c, batch, seq);
  hipStream_t st = (hipStream_t)hip_stream;
  const int dt = c.dtype;
  const size_t es = dtype_size(dt);
  char *ws = (char *)workspace;
  auto at = [&](size_t off) { return ws + off; };
  char *down = at(p.fwd.off_down), *q = at(p.fwd.off_q), *kn = at(p.fwd.off_kn), *vt = at(p.fwd.off_v),
       *o = at(p.fwd.off_o);
  char *cq_raw = at(p.off_cq_raw), *ckv_raw = at(p.off_ckv_raw), *vh = at(p.off_vh), *kh = at(p.off_kh),
       *oh = at(p.off_oh), *doh = at(p.off_doh), *dqh = at(p.off_dqh), *dkh = at(p.off_dkh), *dvh = at(p.off_dvh);
  char *gq = at(p.off_gq), *gkv = at(p.off_gkv), *dcqn = at(p.off_dcqn), *dckv = at(p.off_dckv),
       *ddown = at(p.off_ddown), *wq = at(p.off_wq), *wkv = at(p.off_wkv), *wd = at(p.off_wd);
  int32_t *pos_neg = reinterpret_cast<int32_t *>(at(p.off_pos));
  float *rms = reinterpret_cast<float *>(at(p.off_rms));
  char *tr = at(p.off_tr);
  const int B = (int)batch, S = (int)seq, M = B * S, H = c.num_heads;
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim, dqk = dn + dr;
  const int64_t ld = p.fwd.ld_down;
  const RopeTab tab = make_rope_tab(c.rope, dr);
  const float scale = resolve_scale(c);

  // ---- forward, keeping what the backward reads
  {
    GemmDesc g;
    g.dtype = dt;
    g.M = M;
    g.N = rq + rkv + dr;
    g.K = D;
    g.A = x;
    g.lda = D;
    g.S = M;
    g.H = 1;
    g.nseg = 3;
    g.seg[0] = GemmSeg{w->w_down_q, D, 0, down, rq, ld, 0};
    g.seg[1] = GemmSeg{w->w_down_kv, D, rq, down, rkv, ld, rq};
    g.seg[2] = GemmSeg{w->w_kr, D, rq + rkv, down, dr, ld, rq + rkv};
    MLA_HIP(launch_gemm(g, st), "down projection");
  }
  MLA_HIP(launch_copy_rows(dt, cq_raw, rq, down, ld, M, rq, st), "c_q copy");
  if (w->kv_norm) MLA_HIP(launch_copy_rows(dt, ckv_raw, rkv, down + (size_t)rq * es, ld, M, rkv, st), "c_kv copy");
  MLA_HIP(launch_down_norms(c, w, down, M, ld, st), "rmsnorm");
  MLA_HIP(launch_rope(dt, down + (size_t)(rq + rkv) * es, M, S, (int64_t)S * ld, ld, 1, 0, nullptr, tab, st),
          "rope k_pe");
  {
    GemmDesc g;
    g.dtype = dt;
    g.M = M;
    g.N = H * dqk;
    g.K = rq;
    g.A = down;
    g.lda = ld;
    g.S = S;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_q, rq, 0, q, dn, dqk, 0};
    g.seg[1] = GemmSeg{w->w_qr, rq, H * dn, q, dr, dqk, dn};
    MLA_HIP(launch_gemm(g, st), "q up-projection");
  }
  MLA_HIP(launch_rope(dt, q + (size_t)dn * es, M, S, (int64_t)H * S * dqk, dqk, H, (int64_t)S * dqk, nullptr, tab,
                      st),
          "rope q_pe");
  {
    GemmDesc g;
    g.dtype = dt;
    g.M = M;
    g.N = H * (dn + dv);
    g.K = rkv;
    g.A = down + (size_t)rq * es;
    g.lda = ld;
    g.S = S;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_k, rkv, 0, kn, dn, dn, 0};
    g.seg[1] = GemmSeg{w->w_up_v, rkv, H * dn, vt, dv, dv, 0, 1};  // channel-major for the forward attention
    MLA_HIP(launch_gemm(g, st), "kv up-projection");
    GemmDesc gv = g;  // and row-major per head for the backward
    gv.N = H * dv;
    gv.nseg = 1;
    gv.seg[0] = GemmSeg{w->w_up_v, rkv, 0, vh, dv, dv, 0};
    MLA_HIP(launch_gemm(gv, st), "v up-projection");
  }
  {
    PrefillAttnArgs a;
    a.q = q;
    a.k_nope = kn;
    a.k_pe = down + (size_t)(rq + rkv) * es;
    a.ld_kpe = ld;
    a.vt = vt;
    a.o = o;
    a.B = B;
    a.S = S;
    a.H = H;
    a.scale = scale;
    a.Sk = S;
    MLA_HIP(launch_prefill_attention(dt, dn, dr, dv, a, st), "attention");
  }

  // ---- backward
  // y = o wo^T: dwo = dy^T o, do = dy wo (per head)
  MLA_HIP(bwd_gemm(dt, dy, D, true, o, (int64_t)H * dv, true, grads->wo, (int64_t)H * dv, D, H * dv, M, tr, st),
          "dwo");
  {
    GemmDesc g;
    g.dtype = dt;
    g.M = M;
    g.N = H * dv;
    g.K = D;
    g.A = dy;
    g.lda = D;
    g.b_kn = true;
    g.S = S;
    g.H = H;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->wo, (int64_t)H * dv, 0, doh, dv, dv, 0};
    if (bwd_tr_elems(dt, M, H * dv, D, false, true) > 0) {  // wo^T, K-contiguous
      MLA_HIP(launch_transpose(w->wo, (int64_t)H * dv, D, H * dv, tr, D, st), "wo transpose");
      g.b_kn = false;
      g.seg[0] = GemmSeg{tr, D, 0, doh, dv, dv, 0};
    }
    MLA_HIP(launch_gemm(g, st), "do");
  }
  // attention backward per head on K = [k_nope ‖ k_pe] and the stored o
  MLA_HIP(launch_build_keys(dt, kn, down + (size_t)(rq + rkv) * es, ld, kh, dn, dr, B, S, H, st), "keys");
  MLA_HIP(launch_permute_heads(dt, true, o, (int64_t)H * dv, 0, oh, dv, 0, dv, B, S, H, st), "o per head");
  {
    AttnBwdArgs a;
    a.q = q;
    a.k = kh;
    a.v = vh;
    a.o = oh;
    a.dout = doh;
    a.dq = dqh;
    a.dk = dkh;
    a.dvo = dvh;
    a.lse = reinterpret_cast<float *>(at(p.off_att));
    a.delta = a.lse + (int64_t)M * H;
    a.BH = B * H;
    a.S = S;
    a.dqk = dqk;
    a.dv = dv;
    a.scale = scale;
    MLA_HIP(launch_attention_backward(dt == MLA_DTYPE_BF16 ? BF16 : F32, a, st), "attention backward");
  }
  // RoPE backward (rotation at negated positions) of dq_pe; the shared key's
  // gradient summed over heads, then rotated back, into ddown's k_pe columns
  MLA_HIP(launch_neg_positions(pos_neg, M, S, st), "negated positions");
  MLA_HIP(launch_rope(dt, dqh + (size_t)dn * es, M, S, (int64_t)H * S * dqk, dqk, H, (int64_t)S * dqk, pos_neg, tab,
                      st),
          "rope backward q_pe");
  MLA_HIP(launch_head_sum(dt, dkh, dqk, dn, ddown + (size_t)(rq + rkv) * es, ld, dr, B, S, H, st), "k_pe head sum");
  MLA_HIP(launch_rope(dt, ddown + (size_t)(rq + rkv) * es, M, S, (int64_t)S * ld, ld, 1, 0, pos_neg, tab, st),
          "rope backward k_pe");
  // token-major gradients: gq = [dq_nope ‖ dq_pe_raw], gkv = [dk_nope ‖ dv]
  const int64_t lgq = (int64_t)H * dqk, lgkv = (int64_t)H * (dn + dv);
  MLA_HIP(launch_permute_heads(dt, false, dqh, dqk, 0, gq, lgq, 0, dn, B, S, H, st), "dq_nope rows");
  MLA_HIP(launch_permute_heads(dt, false, dqh, dqk, dn, gq, lgq, H * dn, dr, B, S, H, st), "dq_pe rows");
  MLA_HIP(launch_permute_heads(dt, false, dkh, dqk, 0, gkv, lgkv, 0, dn, B, S, H, st), "dk_nope rows");
  MLA_HIP(launch_permute_heads(dt, false, dvh, dv, 0, gkv, lgkv, H * dn, dv, B, S, H, st), "dv rows");
  // the up-projection weights stacked along their output rows
  MLA_HIP(launch_copy_rows(dt, wq, rq, w->w_up_q, rq, (int64_t)H * dn, rq, st), "stack w_up_q");
  MLA_HIP(launch_copy_rows(dt, wq + (size_t)H * dn * rq * es, rq, w->w_qr, rq, (int64_t)H * dr, rq, st), "stack w_qr");
  MLA_HIP(launch_copy_rows(dt, wkv, rkv, w->w_up_k, rkv, (int64_t)H * dn, rkv, st), "stack w_up_k");
  MLA_HIP(launch_copy_rows(dt, wkv + (size_t)H * dn * rkv * es, rkv, w->w_up_v, rkv, (int64_t)H * dv, rkv, st),
          "stack w_up_v");
  MLA_HIP(launch_copy_rows(dt, wd, D, w->w_down_q, D, rq, D, st), "stack w_down_q");
  MLA_HIP(launch_copy_rows(dt, wd + (size_t)rq * D * es, D, w->w_down_kv, D, rkv, D, st), "stack w_down_kv");
  MLA_HIP(launch_copy_rows(dt, wd + (size_t)(rq + rkv) * D * es, D, w->w_kr, D, dr, D, st), "stack w_kr");
  // q side: dW_uq, dW_qr, dc_qn
  MLA_HIP(bwd_gemm(dt, gq, lgq, true, down, ld, true, grads->w_up_q, rq, H * dn, rq, M, tr, st), "dw_up_q");
  MLA_HIP(bwd_gemm(dt, gq + (size_t)H * dn * es, lgq, true, down, ld, true, grads->w_qr, rq, H * dr, rq, M, tr, st),
          "dw_qr");
  MLA_HIP(bwd_gemm(dt, gq, lgq, false, wq, rq, true, dcqn, rq, M, rq, H * dqk, tr, st), "dc_q");
  // kv side: dW_uk, dW_uv, dc_kv
  MLA_HIP(bwd_gemm(dt, gkv, lgkv, true, down + (size_t)rq * es, ld, true, grads->w_up_k, rkv, H * dn, rkv, M, tr, st),
          "dw_up_k");
  MLA_HIP(bwd_gemm(dt, gkv + (size_t)H * dn * es, lgkv, true, down + (size_t)rq * es, ld, true, grads->w_up_v, rkv,
                     H * dv, rkv, M, tr, st),
          "dw_up_v");
  MLA_HIP(bwd_gemm(dt, gkv, lgkv, false, wkv, rkv, true, dckv, rkv, M, rkv, H * (dn + dv), tr, st), "dc_kv");
  // norms: dc_q (and dc_kv) into ddown's columns, the gains' gradients in fp32
  if (w->kv_norm) {
    MLA_HIP(launch_rmsnorm_backward(dt, ckv_raw, rkv, dckv, rkv, w->kv_norm, M, rkv, c.rms_norm_eps,
                                    ddown + (size_t)rq * es, ld, grads->kv_norm, rms, st),
            "kv norm backward");
  } else {
    MLA_HIP(launch_copy_rows(dt, ddown + (size_t)rq * es, ld, dckv, rkv, M, rkv, st), "dc_kv copy");
  }
  MLA_HIP(launch_rmsnorm_backward(dt, cq_raw, rq, dcqn, rq, w->q_norm, M, rq, c.rms_norm_eps, ddown, ld,
                                  grads->q_norm, rms, st),
          "q norm backward");
  // down projections: dx and the three weights
  MLA_HIP(bwd_gemm(dt, ddown, ld, false, wd, D, true, dx, D, M, D, rq + rkv + dr, tr, st), "dx");
  // the three weights' gradients as one product over ddown's stacked
  // columns [c_q ‖ c_kv ‖ k_pe] (2112 output rows at V3: one well-filled
  // large-tile launch instead of three, the 64-row k_pe one on the general
  // kernel), then split by rows
  const int nd = rq + rkv + dr;
  char *dwd = at(p.off_dwd);
  MLA_HIP(bwd_gemm(dt, ddown, ld, true, x, D, true, dwd, D, nd, D, M, tr, st), "dw_down");
  MLA_HIP(launch_copy_rows(dt, grads->w_down_q, D, dwd, D, rq, D, st), "dw_down_q rows");
  MLA_HIP(launch_copy_rows(dt, grads->w_down_kv, D, dwd + (size_t)rq * D * es, D, rkv, D, st), "dw_down_kv rows");
  MLA_HIP(launch_copy_rows(dt, grads->w_kr, D, dwd + (size_t)(rq + rkv) * D * es, D, dr, D, st), "dw_kr rows");
  return MLA_OK;
}

// ---------------------------------------------------------------- FP8 prefill
// The prefill with its four projection products on block-scaled FP8 (E4M3
// codes, power-of-two scale per 1 x 128 activation tile and 128 x 128
// weight block), attention, norms and RoPE in bf16 / fp32 as in the bf16
// path.  Activations are quantised right after the kernel that produces them.
namespace {

struct Fp8Dims {
  int64_t N[4], K[4];  // down, q up, kv up, out
};

Fp8Dims fp8_dims(const mla_config &c) {
  const int64_t H = c.num_heads;
  Fp8Dims d;
  d.N[0] = c.q_lora_rank + c.kv_lora_rank + c.qk_rope_head_dim;
  d.K[0] = c.hidden_size;
  d.N[1] = H * (c.qk_nope_head_dim + c.qk_rope_head_dim);
  d.K[1] = c.q_lora_rank;
  d.N[2] = H * (c.qk_nope_head_dim + c.v_head_dim);
  d.K[2] = c.kv_lora_rank;
  d.N[3] = c.hidden_size;
  d.K[3] = H * c.v_head_dim;
  return d;
}

mla_status check_fp8_config(const mla_config *cfg) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (cfg->dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_UNSUPPORTED, "the FP8 prefill takes bf16 activations and weights");
  const Fp8Dims d = fp8_dims(*cfg);
  for (int i = 0; i < 4; ++i)
    if (d.K[i] % 128)
      return fail(MLA_ERR_UNSUPPORTED,
                  "FP8 products need reduction lengths that are multiples of 128 (hidden_size, "
                  "q_lora_rank, kv_lora_rank and num_heads * v_head_dim)");
  if (((int64_t)cfg->num_heads * cfg->qk_nope_head_dim) % 256)
    return fail(MLA_ERR_UNSUPPORTED, "num_heads * qk_nope_head_dim must be a multiple of 256 for the FP8 "
                                     "kv up-projection (its v range starts a tile)");
  return MLA_OK;
}

// Bytes of one stacked code matrix and its scale bytes, 256-byte aligned.
size_t fp8_matrix_bytes(int64_t N, int64_t K) {
  return round_up((size_t)N * K, 256) + round_up((size_t)(K / 128) * fp8_scale_pitch(N), 256);
}

mla_status check_fp8_matrix(const mla_fp8_matrix &m, int64_t N, int64_t K, const char *name) {
  if (!m.codes || !m.scales) return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 %s: codes or scales NULL", name);
  if (((uintptr_t)m.codes & 15) || ((uintptr_t)m.scales & 3))
    return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 %s: codes must be 16-byte and scales 4-byte aligned", name);
  if (m.ld < K || m.ld % 16 || m.ld_scales < fp8_scale_pitch(N) || m.ld_scales % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 %s: ld must be >= %lld and a multiple of 16, ld_scales >= "
                "%lld and a multiple of 4", name, (long long)K, (long long)fp8_scale_pitch(N));
  return MLA_OK;
}

struct Fp8PrefillPlan {
  PrefillPlan base;
  int64_t pitch_m;
  size_t off_x8, off_sx, off_cq8, off_scq, off_ckv8, off_sckv, off_o8, off_so, total;
};

Fp8PrefillPlan plan_prefill_fp8(const mla_config &c, int64_t B, int64_t S) {
  Fp8PrefillPlan p;
  p.base = plan_prefill(c, B, S);
  const int64_t M = B * S;
  p.pitch_m = fp8_scale_pitch(M);
  size_t off = p.base.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  const Fp8Dims d = fp8_dims(c);
  p.off_x8 = take((size_t)M * d.K[0]);
  p.off_sx = take((size_t)(d.K[0] / 128) * p.pitch_m);
  p.off_cq8 = take((size_t)M * d.K[1]);
  p.off_scq = take((size_t)(d.K[1] / 128) * p.pitch_m);
  p.off_ckv8 = take((size_t)M * d.K[2]);
  p.off_sckv = take((size_t)(d.K[2] / 128) * p.pitch_m);
  p.off_o8 = take((size_t)M * d.K[3]);
  p.off_so = take((size_t)(d.K[3] / 128) * p.pitch_m);
  p.total = off;
  return p;
}

}  // namespace

mla_status mla_fp8_weights_size(const mla_config *cfg, size_t *bytes) {
  mla_status s = check_fp8_config(cfg);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const Fp8Dims d = fp8_dims(*cfg);
  size_t n = 0;
  for (int i = 0; i < 4; ++i) n += fp8_matrix_bytes(d.N[i], d.K[i]);
  *bytes = n;
  return MLA_OK;
}

mla_status mla_fp8_prepare_weights(const mla_config *cfg, const mla_weights *w, void *buffer,
                                   size_t buffer_bytes, mla_fp8_weights *out, void *hip_stream) {
  mla_status s = check_fp8_config(cfg);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!buffer || !out) return fail(MLA_ERR_INVALID_ARGUMENT, "buffer and out must not be NULL");
  if ((uintptr_t)buffer & 255) return fail(MLA_ERR_INVALID_ARGUMENT, "buffer must be 256-byte aligned");
  size_t need = 0;
  mla_fp8_weights_size(cfg, &need);
  if (buffer_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "buffer has %zu bytes, needs %zu", buffer_bytes, need);
  const mla_config &c = *cfg;
  const Fp8Dims d = fp8_dims(c);
  hipStream_t st = (hipStream_t)hip_stream;
  uint8_t *base = (uint8_t *)buffer;
  mla_fp8_matrix *mats[4] = {&out->down, &out->q_up, &out->kv_up, &out->out};
  size_t off = 0;
  for (int i = 0; i < 4; ++i) {
    mats[i]->codes = base + off;
    mats[i]->ld = d.K[i];
    mats[i]->scales = base + off + round_up((size_t)d.N[i] * d.K[i], 256);
    mats[i]->ld_scales = fp8_scale_pitch(d.N[i]);
    off += fp8_matrix_bytes(d.N[i], d.K[i]);
  }
  const int64_t H = c.num_heads;
  // each source matrix is block-quantised on its own, into its rows of the stack
  struct Part {
    int mat;
    const void *src;
    int64_t rows, row0;
  } parts[] = {
      {0, w->w_down_q, c.q_lora_rank, 0},
      {0, w->w_down_kv, c.kv_lora_rank, c.q_lora_rank},
      {0, w->w_kr, c.qk_rope_head_dim, c.q_lora_rank + c.kv_lora_rank},
      {1, w->w_up_q, H * c.qk_nope_head_dim, 0},
      {1, w->w_qr, H * c.qk_rope_head_dim, H * c.qk_nope_head_dim},
      {2, w->w_up_k, H * c.qk_nope_head_dim, 0},
      {2, w->w_up_v, H * c.v_head_dim, H * c.qk_nope_head_dim},
      {3, w->wo, c.hidden_size, 0},
  };
  for (const Part &pt : parts) {
    mla_fp8_matrix &m = *mats[pt.mat];
    MLA_HIP(launch_fp8_quant_blocks(BF16, pt.src, pt.rows, d.K[pt.mat], d.K[pt.mat],
                                    const_cast<uint8_t *>(m.codes) + pt.row0 * m.ld, m.ld,
                                    const_cast<uint8_t *>(m.scales) + pt.row0, m.ld_scales, st),
            "fp8 weight quantisation");
  }
  return MLA_OK;
}

mla_status mla_prefill_fp8_workspace_size(const mla_config *cfg, int64_t batch, int64_t seq,
                                          size_t *bytes) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if ((s = check_fp8_config(cfg)) != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_prefill_fp8(*cfg, batch, seq).total;
  return MLA_OK;
}

mla_status mla_prefill_forward_fp8(const mla_config *cfg, const mla_weights *w, const mla_fp8_weights *w8,
                                   const void *x, int64_t batch, int64_t seq, void *y, void *latent_out,
                                   void *workspace, size_t workspace_bytes, void *hip_stream) {
  mla_status s = check_prefill_sizes(cfg, batch, seq);
  if (s != MLA_OK) return s;
  if ((s = check_fp8_config(cfg)) != MLA_OK) return s;
  if (!w || !w->q_norm || !aligned16(w->q_norm))
    return fail(MLA_ERR_INVALID_ARGUMENT, "weights->q_norm must be a 16-byte aligned device pointer");
  if (w->kv_norm && !aligned16(w->kv_norm))
    return fail(MLA_ERR_INVALID_ARGUMENT, "weight kv_norm is not 16-byte aligned");
  if (!w8) return fail(MLA_ERR_INVALID_ARGUMENT, "FP8 weights are NULL");
  const mla_config &c = *cfg;
  const Fp8Dims d = fp8_dims(c);
  const mla_fp8_matrix *mats[4] = {&w8->down, &w8->q_up, &w8->kv_up, &w8->out};
  const char *names[4] = {"down", "q_up", "kv_up", "out"};
  for (int i = 0; i < 4; ++i)
    if ((s = check_fp8_matrix(*mats[i], d.N[i], d.K[i], names[i])) != MLA_OK) return s;
  if (!x || !y || !workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, y and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || (latent_out && !aligned16(latent_out)))
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, y, latent_out and workspace must be 16-byte aligned");
  const Fp8PrefillPlan p = plan_prefill_fp8(c, batch, seq);
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, p.total);

  hipStream_t st = (hipStream_t)hip_stream;
  char *ws = (char *)workspace;
  char *down = ws + p.base.off_down, *q = ws + p.base.off_q, *kn = ws + p.base.off_kn,
       *v = ws + p.base.off_v, *o = ws + p.base.off_o;
  uint8_t *x8 = (uint8_t *)(ws + p.off_x8), *sx = (uint8_t *)(ws + p.off_sx);
  uint8_t *cq8 = (uint8_t *)(ws + p.off_cq8), *scq = (uint8_t *)(ws + p.off_scq);
  uint8_t *ckv8 = (uint8_t *)(ws + p.off_ckv8), *sckv = (uint8_t *)(ws + p.off_sckv);
  uint8_t *o8 = (uint8_t *)(ws + p.off_o8), *so = (uint8_t *)(ws + p.off_so);
  const int B = (int)batch, S = (int)seq, M = B * S, H = c.num_heads;
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim, dqk = dn + dr;
  const int64_t ld_down = p.base.ld_down, pm = p.pitch_m;
  const size_t es = 2;
  const RopeTab tab = make_rope_tab(c.rope, dr);
  auto product = [&](int i, const uint8_t *a, const uint8_t *sa, int nseg, const GemmSeg *segs, int Sv,
                     int Hv) {
    Fp8GemmDesc g;
    g.a = a;
    g.sa = sa;
    g.lda = d.K[i];
    g.ld_sa = pm;
    g.b = mats[i]->codes;
    g.sb = mats[i]->scales;
    g.ldb = mats[i]->ld;
    g.ld_sb = mats[i]->ld_scales;
    g.M = M;
    g.N = (int)d.N[i];
    g.K = (int)d.K[i];
    g.S = Sv;
    g.H = Hv;
    g.nseg = nseg;
    for (int k = 0; k < nseg; ++k) g.seg[k] = segs[k];
    return launch_fp8_gemm_seg(g, st);
  };

  // 1. x quantised in 1 x 128 tiles, then [c_q ‖ c_kv ‖ k_pe] (plain rows)
  MLA_MARK(0);
  MLA_HIP(launch_fp8_quant_rows(BF16, x, M, D, D, x8, D, sx, pm, st), "fp8 quantise x");
  {
    const GemmSeg seg{nullptr, 0, 0, down, (int)d.N[0], ld_down, 0};
    MLA_HIP(product(0, x8, sx, 1, &seg, M, 1), "fp8 down projection");
  }
  // 2. RMSNorm(c_q) (and c_kv with kv_norm gains)
  MLA_MARK(1);
  MLA_HIP(launch_down_norms(c, w, down, M, ld_down, st), "rmsnorm");
  // 3. RoPE of the shared key, latent copy
  MLA_MARK(2);
  MLA_HIP(launch_rope(c.dtype, down + (size_t)(rq + rkv) * es, M, S, (int64_t)S * ld_down, ld_down, 1, 0,
                      nullptr, tab, st),
          "rope k_pe");
  if (latent_out)
    MLA_HIP(launch_copy_rows(c.dtype, latent_out, rkv + dr, down + (size_t)rq * es, ld_down, M, rkv + dr, st),
            "latent copy");
  // 4. c_q and c_kv quantised; q = [q_nope ‖ q_pe] per head
  MLA_MARK(3);
  MLA_HIP(launch_fp8_quant_rows(BF16, down, M, rq, ld_down, cq8, rq, scq, pm, st), "fp8 quantise c_q");
  MLA_HIP(launch_fp8_quant_rows(BF16, down + (size_t)rq * es, M, rkv, ld_down, ckv8, rkv, sckv, pm, st),
          "fp8 quantise c_kv");
  {
    const GemmSeg segs[2] = {GemmSeg{nullptr, 0, 0, q, dn, dqk, 0},
                             GemmSeg{nullptr, 0, H * dn, q, dr, dqk, dn}};
    MLA_HIP(product(1, cq8, scq, 2, segs, S, H), "fp8 q up-projection");
  }
  MLA_MARK(4);
  MLA_HIP(launch_rope(c.dtype, q + (size_t)dn * es, M, S, (int64_t)H * S * dqk, dqk, H, (int64_t)S * dqk,
                      nullptr, tab, st),
          "rope q_pe");
  // 5. k_nope head-major, v channel-major
  MLA_MARK(5);
  {
    const GemmSeg segs[2] = {GemmSeg{nullptr, 0, 0, kn, dn, dn, 0},
                             GemmSeg{nullptr, 0, H * dn, v, dv, dv, 0, 1}};
    MLA_HIP(product(2, ckv8, sckv, 2, segs, S, H), "fp8 kv up-projection");
  }
  // 6. causal attention (bf16 operands, fp32 softmax)
  MLA_MARK(6);
  {
    PrefillAttnArgs a;
    a.q = q;
    a.k_nope = kn;
    a.k_pe = down + (size_t)(rq + rkv) * es;
    a.ld_kpe = ld_down;
    a.vt = v;
    a.o = o;
    a.B = B;
    a.S = S;
    a.H = H;
    a.scale = resolve_scale(c);
    a.Sk = S;
    MLA_HIP(launch_prefill_attention(c.dtype, dn, dr, dv, a, st), "attention");
  }
  // 7. o quantised; y = o wo^T
  MLA_MARK(7);
  MLA_HIP(launch_fp8_quant_rows(BF16, o, M, H * dv, (int64_t)H * dv, o8, (int64_t)H * dv, so, pm, st),
          "fp8 quantise o");
  {
    const GemmSeg seg{nullptr, 0, 0, y, D, D, 0};
    MLA_HIP(product(3, o8, so, 1, &seg, M, 1), "fp8 output projection");
  }
  MLA_MARK(8);
  return MLA_OK;
}

static mla_status check_varlen(const mla_config *cfg, int64_t n_seq, int64_t total) {
  if (n_seq < 1 || n_seq > (1 << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "n_seq must be in [1, 2^24]");
  return check_prefill_sizes(cfg, 1, total);
}

mla_status mla_prefill_varlen_workspace_size(const mla_config *cfg, int64_t n_seq,
                                             int64_t total_tokens, size_t *bytes) {
  mla_status s = check_varlen(cfg, n_seq, total_tokens);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_prefill(*cfg, 1, total_tokens, true).total;
  return MLA_OK;
}

mla_status mla_prefill_varlen_forward(const mla_config *cfg, const mla_weights *w, const void *x,
                                      const int32_t *cu_seqlens, int64_t n_seq,
                                      int64_t total_tokens, void *y, void *latent_out,
                                      void *workspace, size_t workspace_bytes,
                                      void *hip_stream) {
  mla_status s = check_varlen(cfg, n_seq, total_tokens);
  if (s != MLA_OK) return s;
  if (!cu_seqlens) return fail(MLA_ERR_INVALID_ARGUMENT, "cu_seqlens must not be NULL");
  if (((uintptr_t)cu_seqlens & 3) != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  return prefill_common(cfg, w, x, 1, total_tokens, y, latent_out, workspace, workspace_bytes,
                        hip_stream, cu_seqlens, n_seq);
}

mla_status mla_decode_workspace_size(const mla_config *cfg, int64_t batch, int64_t cache_capacity,
                                     size_t *bytes) {
  mla_status s = check_decode_sizes(cfg, batch, cache_capacity);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_decode(*cfg, batch).total;
  return MLA_OK;
}

// ------------------------------------------------------------ chunked prefill
// q_len new tokens per sequence against a latent cache, expanded form: the
// cached rows (prefix and the new rows) of every usable sequence are packed
// into one key stream, up-projected to per-head keys and values, and the
// prefill attention runs each query over its own sequence's keys.
struct ChunkPlan {
  int64_t ld_down, kmax;
  size_t off_down, off_q, off_o, off_kstream, off_kn, off_v, off_lens, off_kofs, off_lo, off_hi,
      off_pos, off_valid, off_gemm, gemm_bytes, total;
};

static ChunkPlan plan_chunk(const mla_config &c, int64_t B, int64_t T, int64_t max_keys) {
  const size_t es = dtype_size(c.dtype);
  const int64_t M = B * T, H = c.num_heads, W = c.kv_lora_rank + c.qk_rope_head_dim;
  ChunkPlan p;
  p.ld_down = (int64_t)round_up(c.q_lora_rank + W, 8);
  p.kmax = (int64_t)round_up((size_t)max_keys, 8);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  p.off_down = take((size_t)M * p.ld_down * es);
  p.off_q = take((size_t)M * H * (c.qk_nope_head_dim + c.qk_rope_head_dim) * es);
  p.off_o = take((size_t)M * H * c.v_head_dim * es);
  p.off_kstream = take((size_t)p.kmax * W * es);
  p.off_kn = take((size_t)p.kmax * H * c.qk_nope_head_dim * es);
  p.off_v = take((size_t)p.kmax * H * c.v_head_dim * es);
  p.off_lens = take((size_t)B * sizeof(int32_t));
  p.off_kofs = take((size_t)(B + 1) * sizeof(int32_t));
  p.off_lo = take((size_t)M * sizeof(int32_t));
  p.off_hi = take((size_t)M * sizeof(int32_t));
  p.off_pos = take((size_t)M * sizeof(int32_t));
  p.off_valid = take((size_t)M * sizeof(int32_t));
  // fp32 split-K partials of the projections with few rows
  const int dt = c.dtype, D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dqk = c.qk_nope_head_dim + c.qk_rope_head_dim;
  p.gemm_bytes = std::max(std::max(gemm_scratch_bytes(dt, (int)M, rq + (int)W, D, 1),
                                   gemm_scratch_bytes(dt, (int)M, (int)H * dqk, rq, 1)),
                          std::max(gemm_scratch_bytes(dt, (int)M, D, (int)H * c.v_head_dim, 1),
                                   gemm_scratch_bytes(dt, (int)p.kmax,
                                                      (int)H * (c.qk_nope_head_dim + c.v_head_dim),
                                                      rkv, 1)));
  p.off_gemm = take(p.gemm_bytes);
  p.total = off;
  return p;
}

static mla_status check_chunk(const mla_config *cfg, int64_t B, int64_t T, int64_t cap,
                              int64_t max_keys) {
  mla_status s = check_config(cfg);
  if (s != MLA_OK) return s;
  if (B < 1 || B > 4096) return fail(MLA_ERR_INVALID_ARGUMENT, "batch must be in [1, 4096]");
  if (T < 1 || T > cap) return fail(MLA_ERR_INVALID_ARGUMENT, "q_len must be in [1, cache_capacity]");
  if (B * cap > (1LL << 30) || B * T > (1LL << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch x cache_capacity or batch x q_len is too large");
  if (max_keys < T || max_keys > (1LL << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "max_keys must be in [q_len, 2^24]");
  if (!prefill_instance(*cfg))
    return fail(MLA_ERR_UNSUPPORTED,
                "head dims (nope %d, rope %d, v %d) are not instantiated; supported: "
                "(16,8,16), (64,32,64), (128,64,128)",
                cfg->qk_nope_head_dim, cfg->qk_rope_head_dim, cfg->v_head_dim);
  return MLA_OK;
}

mla_status mla_prefill_chunk_workspace_size(const mla_config *cfg, int64_t batch, int64_t q_len,
                                            int64_t cache_capacity, int64_t max_keys,
                                            size_t *bytes) {
  mla_status s = check_chunk(cfg, batch, q_len, cache_capacity, max_keys);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_chunk(*cfg, batch, q_len, max_keys).total;
  return MLA_OK;
}

mla_status mla_prefill_chunk(const mla_config *cfg, const mla_weights *w, const void *x,
                             int64_t batch, int64_t q_len, void *latent_cache,
                             int64_t cache_capacity, const int32_t *cache_lens, int64_t max_keys,
                             void *y, void *workspace, size_t workspace_bytes, void *hip_stream) {
  mla_status s = check_chunk(cfg, batch, q_len, cache_capacity, max_keys);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!x || !y || !workspace || !latent_cache || !cache_lens)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "x, y, latent_cache, cache_lens and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || !aligned16(latent_cache) ||
      ((uintptr_t)cache_lens & 3) != 0)
    return fail(MLA_ERR_INVALID_ARGUMENT, "x, y, latent_cache and workspace must be 16-byte "
                                          "aligned, cache_lens 4-byte aligned");
  const mla_config &c = *cfg;
  const ChunkPlan p = plan_chunk(c, batch, q_len, max_keys);
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, p.total);

  hipStream_t st = (hipStream_t)hip_stream;
  const size_t es = dtype_size(c.dtype);
  char *ws = (char *)workspace;
  char *down = ws + p.off_down, *q = ws + p.off_q, *o = ws + p.off_o;
  char *kst = ws + p.off_kstream, *kn = ws + p.off_kn, *v = ws + p.off_v;
  int32_t *lens_eff = reinterpret_cast<int32_t *>(ws + p.off_lens);
  int32_t *kofs = reinterpret_cast<int32_t *>(ws + p.off_kofs);
  int32_t *lo = reinterpret_cast<int32_t *>(ws + p.off_lo);
  int32_t *hi = reinterpret_cast<int32_t *>(ws + p.off_hi);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + p.off_pos);
  int32_t *valid = reinterpret_cast<int32_t *>(ws + p.off_valid);
  const int B = (int)batch, T = (int)q_len, M = B * T, H = c.num_heads;
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim;
  const int dqk = dn + dr, W = rkv + dr;
  const int K = (int)p.kmax;
  const RopeTab tab = make_rope_tab(c.rope, dr);

  // usable sequences, packed key offsets, per-query key ranges and positions
  MLA_HIP(launch_chunk_index(cache_lens, B, T, cache_capacity, max_keys, lens_eff, kofs, lo, hi, pos,
                             valid, st),
          "chunk index");
  {  // [c_q ‖ c_kv ‖ k_pe] = x [w_down_q; w_down_kv; w_kr]^T
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = M;
    g.N = rq + W;
    g.K = D;
    g.A = x;
    g.lda = D;
    g.S = M;
    g.H = 1;
    g.nseg = 3;
    g.seg[0] = GemmSeg{w->w_down_q, D, 0, down, rq, p.ld_down, 0};
    g.seg[1] = GemmSeg{w->w_down_kv, D, rq, down, rkv, p.ld_down, rq};
    g.seg[2] = GemmSeg{w->w_kr, D, rq + rkv, down, dr, p.ld_down, rq + rkv};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "down projection");
  }
  MLA_HIP(launch_down_norms(c, w, down, M, p.ld_down, st), "rmsnorm");
  MLA_HIP(launch_rope(c.dtype, down + (size_t)(rq + rkv) * es, M, M, (int64_t)M * p.ld_down,
                      p.ld_down, 1, 0, pos, tab, st),
          "rope k_pe");
  // the new latent rows go to cache rows L_b .. L_b + T - 1 (usable sequences)
  MLA_HIP(launch_cache_append(c.dtype, latent_cache, cache_capacity, lens_eff, T,
                              down + (size_t)rq * es, p.ld_down, B, W, st),
          "cache append");
  {  // q = [q_nope ‖ q_pe] per head over all M queries
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = M;
    g.N = H * dqk;
    g.K = rq;
    g.A = down;
    g.lda = p.ld_down;
    g.S = M;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_q, rq, 0, q, dn, dqk, 0};
    g.seg[1] = GemmSeg{w->w_qr, rq, H * dn, q, dr, dqk, dn};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "q up-projection");
  }
  MLA_HIP(launch_rope(c.dtype, q + (size_t)dn * es, M, M, (int64_t)H * M * dqk, dqk, H,
                      (int64_t)M * dqk, pos, tab, st),
          "rope q_pe");
  // key stream: every usable sequence's cache rows 0 .. L_b + T - 1, packed
  MLA_HIP(launch_gather_keys(c.dtype, kst, K, latent_cache, cache_capacity, W, kofs, B, st),
          "key gather");
  {  // k_nope [1, H, K, d_n] and v channel-major [1, H, d_v, K]
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = K;
    g.N = H * (dn + dv);
    g.K = rkv;
    g.A = kst;
    g.lda = W;
    g.S = K;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_k, rkv, 0, kn, dn, dn, 0};
    g.seg[1] = GemmSeg{w->w_up_v, rkv, H * dn, v, dv, dv, 0, 1};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "kv up-projection");
  }
  {
    PrefillAttnArgs a;
    a.q = q;
    a.k_nope = kn;
    a.k_pe = kst + (size_t)rkv * es;
    a.ld_kpe = W;
    a.vt = v;
    a.o = o;
    a.B = 1;
    a.S = M;
    a.H = H;
    a.scale = resolve_scale(c);
    a.kv_lo = lo;
    a.kv_hi = hi;
    a.valid = valid;
    a.Sk = K;
    MLA_HIP(launch_prefill_attention(c.dtype, dn, dr, dv, a, st), "attention");
  }
  {  // y = o wo^T
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = M;
    g.N = D;
    g.K = H * dv;
    g.A = o;
    g.lda = (int64_t)H * dv;
    g.S = M;
    g.H = 1;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->wo, (int64_t)H * dv, 0, y, D, D, 0};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "output projection");
  }
  return MLA_OK;
}

mla_status mla_decode_multi_workspace_size(const mla_config *cfg, int64_t batch, int64_t q_len,
                                           int64_t cache_capacity, size_t *bytes) {
  mla_status s = check_decode_sizes(cfg, batch, cache_capacity, q_len);
  if (s != MLA_OK) return s;
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = plan_decode(*cfg, batch, q_len).total;
  return MLA_OK;
}

mla_status mla_decode_layout_of(const mla_config *cfg, int64_t batch, int64_t cache_capacity,
                                mla_decode_layout *layout) {
  mla_status s = check_decode_sizes(cfg, batch, cache_capacity);
  if (s != MLA_OK) return s;
  if (!layout) return fail(MLA_ERR_INVALID_ARGUMENT, "layout is NULL");
  const DecodePlan p = plan_decode(*cfg, batch);
  layout->c_q = p.off_down;
  layout->c_kv = p.off_down + (size_t)cfg->q_lora_rank * dtype_size(cfg->dtype);
  layout->q = p.off_qn;
  layout->q_lat = p.off_qlat;
  layout->o_lat = p.off_olat;
  layout->o = p.off_o;
  layout->ld_down = p.ld_down;
  layout->n_splits = p.n_blocks;
  layout->split_len = 0;
  layout->total = p.total;
  return MLA_OK;
}

namespace {
mla_status decode_impl(const mla_config *cfg, const mla_weights *w, const void *x, int64_t batch,
                       int64_t q_len, void *latent_cache, int64_t cache_capacity,
                       const int32_t *cache_lens, void *y, void *workspace,
                       size_t workspace_bytes, void *hip_stream) {
  mla_status s = check_decode_sizes(cfg, batch, cache_capacity, q_len);
  if (s != MLA_OK) return s;
  if ((s = check_weights(w)) != MLA_OK) return s;
  if (!x || !y || !workspace || !latent_cache || !cache_lens)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "x, latent_cache, cache_lens, y and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || !aligned16(latent_cache))
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "x, y, latent_cache and workspace must be 16-byte aligned");
  const mla_config &c = *cfg;
  const DecodePlan p = plan_decode(c, batch, q_len);
  if (workspace_bytes < p.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                workspace_bytes, p.total);

  hipStream_t st = (hipStream_t)hip_stream;
  const int T = (int)q_len;
  const size_t es = dtype_size(c.dtype);
  char *ws = (char *)workspace;
  char *down = ws + p.off_down;
  char *qn = ws + p.off_qn;
  char *qlat = ws + p.off_qlat;
  char *olat = ws + p.off_olat;
  char *o = ws + p.off_o;
  // B token rows (sequence b's token t is row b*T + t); Bs sequences
  const int Bs = (int)batch, B = Bs * T, H = c.num_heads;
  const int D = c.hidden_size, rq = c.q_lora_rank, rkv = c.kv_lora_rank;
  const int dn = c.qk_nope_head_dim, dr = c.qk_rope_head_dim, dv = c.v_head_dim;
  const int wl = rkv + dr;  // latent row width
  const RopeTab tab = make_rope_tab(c.rope, dr);
  // position of each token row: lens[b] + t (the lengths themselves at T = 1)
  const int32_t *pos = cache_lens;
  if (T > 1) {
    int32_t *pw = (int32_t *)(ws + p.off_pos);
    MLA_HIP(launch_decode_positions(cache_lens, Bs, T, pw, st), "decode positions");
    pos = pw;
  }

  // 1. down projections of the new tokens
  MLA_MARK(0);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = B;
    g.N = rq + rkv + dr;
    g.K = D;
    g.A = x;
    g.lda = D;
    g.S = B;
    g.H = 1;
    g.nseg = 3;
    g.seg[0] = GemmSeg{w->w_down_q, D, 0, down, rq, p.ld_down, 0};
    g.seg[1] = GemmSeg{w->w_down_kv, D, rq, down, rkv, p.ld_down, rq};
    g.seg[2] = GemmSeg{w->w_kr, D, rq + rkv, down, dr, p.ld_down, rq + rkv};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "decode down projection");
  }
  MLA_MARK(1);
  MLA_HIP(launch_down_norms(c, w, down, B, p.ld_down, st), "decode rmsnorm");
  // 2. RoPE of the new key at position lens[b], then append [c_kv ‖ k_pe] at row lens[b]
  MLA_MARK(2);
  MLA_HIP(launch_rope(c.dtype, down + (size_t)(rq + rkv) * es, B, B, 0, p.ld_down, 1, 0, pos,
                      tab, st),
          "decode rope k_pe");
  MLA_HIP(launch_cache_append(c.dtype, latent_cache, cache_capacity, cache_lens, T,
                              down + (size_t)rq * es, p.ld_down, Bs, wl, st),
          "cache append");
  // 3. q_nope per head, q_pe straight into the absorbed query rows, RoPE of q_pe
  MLA_MARK(3);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = B;
    g.N = H * (dn + dr);
    g.K = rq;
    g.A = down;
    g.lda = p.ld_down;
    g.S = 1;
    g.H = H;
    g.nseg = 2;
    g.seg[0] = GemmSeg{w->w_up_q, rq, 0, qn, dn, dn, 0};
    g.seg[1] = GemmSeg{w->w_qr, rq, H * dn, qlat, dr, wl, rkv};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "decode q up-projection");
  }
  MLA_MARK(4);
  MLA_HIP(launch_rope(c.dtype, qlat + (size_t)rkv * es, B, B, 0, (int64_t)H * wl, H, wl, pos,
                      tab, st),
          "decode rope q_pe");
  // 4. absorb: q_lat[b, h] = w_up_k_h^T q_nope[b, h]   (batched over heads)
  MLA_MARK(5);
  if (c.dtype == MLA_DTYPE_BF16 && dn == 128) {
    MLA_HIP(launch_absorb(c.dtype, dn, rkv, H, B, qn, (int64_t)H * dn, w->w_up_k, qlat,
                          (int64_t)H * wl, wl, st),
            "absorb");
  } else {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = B;
    g.N = rkv;
    g.K = dn;
    g.batch = H;
    g.A = qn;
    g.lda = (int64_t)H * dn;
    g.strideA = dn;
    g.b_kn = true;
    g.strideB = (int64_t)dn * rkv;
    g.strideC = wl;
    g.S = B;
    g.H = 1;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->w_up_k, rkv, 0, qlat, rkv, (int64_t)H * wl, 0};
    MLA_HIP(launch_gemm(g, st), "absorb");
  }
  // 5. latent attention over rows 0..lens[b], split evenly over workgroups, merged
  MLA_MARK(6);
  {
    DecodeAttnArgs a;
    a.q_lat = qlat;
    a.cache = latent_cache;
    a.lens = cache_lens;
    a.o_lat = olat;
    a.part_o = ws + p.off_po;
    a.part_ml = (float *)(ws + p.off_pml);
    a.cap = cache_capacity;
    a.B = Bs;
    a.H = T * H;  // query heads: token t's head h is t*H + h
    a.q_len = T;
    a.heads_per_tok = H;
    a.n_blocks = p.n_blocks;
    a.scale = resolve_scale(c);
    MLA_HIP(launch_decode_attention(c.dtype, rkv, dr, a, st), "decode attention");
    MLA_MARK(7);
    MLA_HIP(launch_decode_merge(c.dtype, rkv, a, st), "decode merge");
  }
  // 6. un-absorb: o[b, h] = w_up_v_h o_lat[b, h]   (batched over heads)
  MLA_MARK(8);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = B;
    g.N = dv;
    g.K = rkv;
    g.batch = H;
    g.A = olat;
    g.lda = (int64_t)H * rkv;
    g.strideA = rkv;
    g.strideB = (int64_t)dv * rkv;
    g.strideC = dv;
    g.S = B;
    g.H = 1;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->w_up_v, rkv, 0, o, dv, (int64_t)H * dv, 0};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "un-absorb");
  }
  // 7. y = o wo^T
  MLA_MARK(9);
  {
    GemmDesc g;
    g.dtype = c.dtype;
    g.M = B;
    g.N = D;
    g.K = H * dv;
    g.A = o;
    g.lda = (int64_t)H * dv;
    g.S = B;
    g.H = 1;
    g.nseg = 1;
    g.seg[0] = GemmSeg{w->wo, (int64_t)H * dv, 0, y, D, D, 0};
    g.workspace = ws + p.off_gemm;
    g.workspace_bytes = p.gemm_bytes;
    MLA_HIP(launch_gemm(g, st), "decode output projection");
  }
  MLA_MARK(10);
  return MLA_OK;
}
}  // namespace

mla_status mla_decode_absorbed(const mla_config *cfg, const mla_weights *w, const void *x,
                               int64_t batch, void *latent_cache, int64_t cache_capacity,
                               const int32_t *cache_lens, void *y, void *workspace,
                               size_t workspace_bytes, void *hip_stream) {
  return decode_impl(cfg, w, x, batch, 1, latent_cache, cache_capacity, cache_lens, y, workspace,
                     workspace_bytes, hip_stream);
}

mla_status mla_decode_absorbed_multi(const mla_config *cfg, const mla_weights *w, const void *x,
                                     int64_t batch, int64_t q_len, void *latent_cache,
                                     int64_t cache_capacity, const int32_t *cache_lens, void *y,
                                     void *workspace, size_t workspace_bytes, void *hip_stream) {
  return decode_impl(cfg, w, x, batch, q_len, latent_cache, cache_capacity, cache_lens, y,
                     workspace, workspace_bytes, hip_stream);
}

mla_status mla_attention_backward_workspace_size(int64_t batch_heads, int64_t seq, size_t *bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (batch_heads < 0 || seq < 0 || batch_heads * seq > INT32_MAX)
    return fail(MLA_ERR_INVALID_ARGUMENT, "batch_heads and seq must be >= 0 with a product below 2^31");
  *bytes = (size_t)batch_heads * seq * 2 * sizeof(float);
  return MLA_OK;
}

}  // extern "C"

namespace {
// Checks shared by mla_attention_backward and its allocation-free variant;
// *need receives the scratch bytes the call uses.
mla_status check_attention_backward(int32_t dtype, int64_t batch_heads, int64_t seq, int32_t d_qk, int32_t d_v,
                                    float scale, const void *const *ptrs, int n_ptrs, size_t *need) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dtype %d is neither 0 (fp32) nor 1 (bf16)", dtype);
  mla_status s = mla_attention_backward_workspace_size(batch_heads, seq, need);
  if (s != MLA_OK) return s;
  if (d_qk < 8 || d_qk > 256 || d_qk % 8 || d_v < 8 || d_v > 256 || d_v % 8)
    return fail(MLA_ERR_INVALID_ARGUMENT, "d_qk and d_v must be multiples of 8 in [8, 256]");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(MLA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (batch_heads * seq == 0) return MLA_OK;
  for (int i = 0; i < n_ptrs; ++i) {
    if (!ptrs[i]) return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor or the workspace is NULL");
    if ((uintptr_t)ptrs[i] % 16)
      return fail(MLA_ERR_INVALID_ARGUMENT, "tensors and workspace must be 16-byte aligned");
  }
  return MLA_OK;
}

mla_status run_attention_backward(int32_t dtype, int64_t batch_heads, int64_t seq, int32_t d_qk, int32_t d_v,
                                  float scale, const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, void *dq, void *dk, void *dv, float *row_stats,
                                  void *hip_stream) {
  AttnBwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dvo = dv;
  a.lse = row_stats;
  a.delta = a.lse + batch_heads * seq;
  a.BH = (int)batch_heads; a.S = (int)seq; a.dqk = d_qk; a.dv = d_v; a.scale = scale;
  MLA_HIP(launch_attention_backward(dtype == MLA_DTYPE_BF16 ? BF16 : F32, a, (hipStream_t)hip_stream),
          "attention backward");
  return MLA_OK;
}

// ---- allocation-free attention backward (scratch array) ----
// Scratch of the allocation-free attention backward: the rows' log-sum-exp
// and rowsum(dO * O), 8 bytes per row, for at most 2^21 rows (16 MB).  Each
// GPU the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address (on the host it stands for
// the symbol, not for device memory): the device address comes from
// hipGetSymbolAddress, once per device, and is passed to the kernels.
constexpr int64_t kNoallocMaxRows = (int64_t)1 << 21;
static __device__ __align__(256) float scratch[2 * kNoallocMaxRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use with
// the device current), or an error status.
mla_status scratch_of_device(int dev, float **out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_INVALID_ARGUMENT, "device %d is beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    MLA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}
// ---- end of the allocation-free scratch ----
}  // namespace

extern "C" {

mla_status mla_attention_backward(int32_t dtype, int64_t batch_heads, int64_t seq, int32_t d_qk, int32_t d_v,
                                  float scale, const void *q, const void *k, const void *v, const void *o,
                                  const void *dout, void *dq, void *dk, void *dv, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
  size_t need = 0;
  const void *ptrs[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  mla_status s = check_attention_backward(dtype, batch_heads, seq, d_qk, d_v, scale, ptrs, 9, &need);
  if (s != MLA_OK || batch_heads * seq == 0) return s;
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
  return run_attention_backward(dtype, batch_heads, seq, d_qk, d_v, scale, q, k, v, o, dout, dq, dk, dv,
                                reinterpret_cast<float *>(workspace), hip_stream);
}

// ---- allocation-free attention backward (entry points) ----
int64_t mla_attention_backward_noalloc_max_rows(void) { return kNoallocMaxRows; }

mla_status mla_attention_backward_noalloc(int32_t dtype, int64_t batch_heads, int64_t seq, int32_t d_qk,
                                          int32_t d_v, float scale, const void *q, const void *k,
                                          const void *v, const void *o, const void *dout, void *dq, void *dk,
                                          void *dv, void *hip_stream) {
  size_t need = 0;
  const void *ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  mla_status s = check_attention_backward(dtype, batch_heads, seq, d_qk, d_v, scale, ptrs, 8, &need);
  if (s != MLA_OK || batch_heads * seq == 0) return s;
  if (batch_heads * seq > kNoallocMaxRows)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "batch_heads x seq = %lld rows exceeds the %lld rows of the built-in scratch",
                (long long)(batch_heads * seq), (long long)kNoallocMaxRows);
  int dev = -1;
  MLA_HIP(hipGetDevice(&dev), "current device");
  if (hip_stream) {
    hipDevice_t sdev = -1;
    MLA_HIP(hipStreamGetDevice((hipStream_t)hip_stream, &sdev), "stream device");
    if (sdev != dev)
      return fail(MLA_ERR_INVALID_ARGUMENT, "the stream belongs to device %d, not the current device %d",
                  (int)sdev, dev);
  }
  float *scr = nullptr;
  if ((s = scratch_of_device(dev, &scr)) != MLA_OK) return s;
  return run_attention_backward(dtype, batch_heads, seq, d_qk, d_v, scale, q, k, v, o, dout, dq, dk, dv, scr,
                                hip_stream);
}

// ---- end of the allocation-free entry points ----

mla_status mla_rmsnorm_backward_workspace_size(int64_t rows, int32_t n, size_t *bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (rows < 0 || rows > INT32_MAX) return fail(MLA_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1]");
  if (n < 1 || n > (1 << 20)) return fail(MLA_ERR_INVALID_ARGUMENT, "n must be in [1, 2^20]");
  *bytes = rmsnorm_backward_scratch_floats(rows, n) * sizeof(float);
  return MLA_OK;
}

mla_status mla_rmsnorm_backward(int32_t dtype, const void *x, const void *dy, const void *g, int64_t rows,
                                int32_t n, float eps, void *dx, float *dg, void *workspace, size_t workspace_bytes,
                                void *hip_stream) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dtype %d is neither 0 (fp32) nor 1 (bf16)", dtype);
  if (rows < 0 || rows > INT32_MAX) return fail(MLA_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^31 - 1]");
  if (n < 1 || n > (1 << 20)) return fail(MLA_ERR_INVALID_ARGUMENT, "n must be in [1, 2^20]");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (rows == 0) return MLA_OK;
  const void *ptrs[] = {x, dy, g, dx, dg, workspace};
  for (const void *p : ptrs) {
    if (!p) return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor or the workspace is NULL");
    if ((uintptr_t)p % 4) return fail(MLA_ERR_INVALID_ARGUMENT, "tensors and workspace must be 4-byte aligned");
  }
  const size_t need = rmsnorm_backward_scratch_floats(rows, n) * sizeof(float);
  if (workspace_bytes < need) return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", need);
  MLA_HIP(launch_rmsnorm_backward(dtype == MLA_DTYPE_BF16 ? BF16 : F32, x, n, dy, n, g, rows, n, eps, dx, n, dg,
                                  reinterpret_cast<float *>(workspace), (hipStream_t)hip_stream),
          "rmsnorm backward");
  return MLA_OK;
}

int64_t mla_fp8_scale_pitch(int64_t rows) { return rows < 0 ? -1 : fp8_scale_pitch(rows); }

static mla_status check_fp8_quant(const void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ldx,
                                  const uint8_t *q, int64_t ldq, const uint8_t *sexp, int64_t ld_sexp,
                                  int64_t q_align) {
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dtype %d is neither 0 (fp32) nor 1 (bf16)", dtype);
  if (rows < 0 || rows > (1 << 24)) return fail(MLA_ERR_INVALID_ARGUMENT, "rows must be in [0, 2^24]");
  if (cols < 128 || cols % 128 || cols > (1 << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "cols must be a positive multiple of 128 (at most 2^24)");
  if (ldx < cols || ldq < cols) return fail(MLA_ERR_INVALID_ARGUMENT, "ldx and ldq must be >= cols");
  if (ld_sexp < rows) return fail(MLA_ERR_INVALID_ARGUMENT, "ld_sexp must be >= rows");
  if (ldq % q_align) return fail(MLA_ERR_INVALID_ARGUMENT, "ldq must be a multiple of %lld", (long long)q_align);
  if (rows == 0) return MLA_OK;
  if (!x || !q || !sexp) return fail(MLA_ERR_INVALID_ARGUMENT, "x, q and sexp must not be NULL");
  if ((uintptr_t)x % dtype_size(dtype)) return fail(MLA_ERR_INVALID_ARGUMENT, "x is not aligned to its element size");
  if ((uintptr_t)q % q_align) return fail(MLA_ERR_INVALID_ARGUMENT, "q must be %lld-byte aligned", (long long)q_align);
  return MLA_OK;
}

mla_status mla_fp8_quantize_rows(const void *x, int32_t dtype, int64_t rows, int64_t cols, int64_t ldx, uint8_t *q,
                                 int64_t ldq, uint8_t *sexp, int64_t ld_sexp, void *hip_stream) {
  mla_status s = check_fp8_quant(x, dtype, rows, cols, ldx, q, ldq, sexp, ld_sexp, 2);
  if (s != MLA_OK || rows == 0) return s;
  MLA_HIP(launch_fp8_quant_rows(dtype, x, rows, cols, ldx, q, ldq, sexp, ld_sexp, (hipStream_t)hip_stream),
          "fp8 quantize rows");
  return MLA_OK;
}

mla_status mla_fp8_quantize_blocks(const void *w, int32_t dtype, int64_t rows, int64_t cols, int64_t ldw,
                                   uint8_t *q, int64_t ldq, uint8_t *sexp, int64_t ld_sexp, void *hip_stream) {
  mla_status s = check_fp8_quant(w, dtype, rows, cols, ldw, q, ldq, sexp, ld_sexp, 16);
  if (s != MLA_OK || rows == 0) return s;
  MLA_HIP(launch_fp8_quant_blocks(dtype, w, rows, cols, ldw, q, ldq, sexp, ld_sexp, (hipStream_t)hip_stream),
          "fp8 quantize blocks");
  return MLA_OK;
}

mla_status mla_fp8_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa, const uint8_t *b,
                        int64_t ldb, const uint8_t *sb, int64_t ld_sb, void *c, int32_t c_dtype, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void *hip_stream) {
  if (c_dtype != MLA_DTYPE_F32 && c_dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "c_dtype %d is neither 0 (fp32) nor 1 (bf16)", c_dtype);
  if (M < 0 || M > (1 << 24) || N < 1 || N > (1 << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "M must be in [0, 2^24] and N in [1, 2^24]");
  if (K < 128 || K % 128 || K > (1 << 24))
    return fail(MLA_ERR_INVALID_ARGUMENT, "K must be a positive multiple of 128 (at most 2^24)");
  if (lda < K || ldb < K || lda % 16 || ldb % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "lda and ldb must be >= K and multiples of 16");
  if (ld_sa < fp8_scale_pitch(M) || ld_sb < fp8_scale_pitch(N) || ld_sa % 4 || ld_sb % 4)
    return fail(MLA_ERR_INVALID_ARGUMENT,
                "ld_sa / ld_sb must be multiples of 4 and at least mla_fp8_scale_pitch(M) / (N)");
  if (ldc < N) return fail(MLA_ERR_INVALID_ARGUMENT, "ldc must be >= N");
  if (c_dtype == MLA_DTYPE_BF16 && (N % 8 || ldc % 8))
    return fail(MLA_ERR_INVALID_ARGUMENT, "bf16 C needs N and ldc multiples of 8");
  if (M == 0) return MLA_OK;
  if (!a || !b || !sa || !sb || !c) return fail(MLA_ERR_INVALID_ARGUMENT, "a, sa, b, sb and c must not be NULL");
  if ((uintptr_t)a % 16 || (uintptr_t)b % 16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a and b must be 16-byte aligned");
  if ((uintptr_t)sa % 4 || (uintptr_t)sb % 4) return fail(MLA_ERR_INVALID_ARGUMENT, "sa and sb must be 4-byte aligned");
  if ((uintptr_t)c % (c_dtype == MLA_DTYPE_BF16 ? 16 : 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "c is not aligned (16 bytes for bf16, 4 for fp32)");
  MLA_HIP(launch_fp8_gemm(a, lda, sa, ld_sa, b, ldb, sb, ld_sb, c, c_dtype == MLA_DTYPE_F32 ? F32 : BF16, ldc,
                          (int)M, (int)N, (int)K, (hipStream_t)hip_stream),
          "fp8 gemm");
  return MLA_OK;
}

mla_status mla_rope_apply(void *x, int32_t dtype, int64_t n_tokens, int32_t n_heads,
                          int32_t rope_dim, int64_t token_stride, int64_t head_stride,
                          const int32_t *positions, const mla_rope_params *params,
                          void *hip_stream) {
  if (!x) return fail(MLA_ERR_INVALID_ARGUMENT, "x is NULL");
  if (dtype != MLA_DTYPE_F32 && dtype != MLA_DTYPE_BF16)
    return fail(MLA_ERR_INVALID_ARGUMENT, "dtype %d is neither 0 (fp32) nor 1 (bf16)", dtype);
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0");
  if (n_heads < 1) return fail(MLA_ERR_INVALID_ARGUMENT, "n_heads must be >= 1");
  mla_status s = check_rope(params, rope_dim);
  if (s != MLA_OK) return s;
  if (!positions && n_tokens > 0) return fail(MLA_ERR_INVALID_ARGUMENT, "positions is NULL");
  if (((uintptr_t)x) % dtype_size(dtype))
    return fail(MLA_ERR_INVALID_ARGUMENT, "x is not aligned to its element size");
  const RopeTab tab = make_rope_tab(*params, rope_dim);
  MLA_HIP(launch_rope(dtype, x, n_tokens, n_tokens > 0 ? n_tokens : 1, 0, token_stride, n_heads,
                      head_stride, positions, tab, (hipStream_t)hip_stream),
          "rope");
  return MLA_OK;
}

}  // extern "C"
