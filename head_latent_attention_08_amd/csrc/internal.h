// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum DType { F32 = 0, BF16 = 1 };

inline size_t dtype_size(int dt) { return dt == BF16 ? 2 : 4; }

// One contiguous range of output columns [n_begin, next n_begin) of a GEMM:
// where its B rows come from and where its results go.  Output column n of
// the range maps to head h = (n - n_begin) / dh and channel d = (n - n_begin)
// % dh, and output row m to (b, s) = (m / S, m % S); the element lands at
//   C + ((b * H + h) * S + s) * ld + off + d              (tr == 0)
//   C + ((b * H + h) * dh + d) * S + s                    (tr == 1, channel-major)
// With H = 1 and dh >= width the first is a plain row-major store with row
// pitch ld.
struct GemmSeg {
  const void *B;
  int64_t ldb;
  int n_begin;
  void *C;
  int dh;
  int64_t ld;
  int off;
  int tr = 0;
};

struct GemmDesc {
  int dtype = BF16;
  int M = 0, N = 0, K = 0;
  int batch = 1;
  const void *A = nullptr;
  int64_t lda = 0, strideA = 0;  // elements
  int64_t strideB = 0, strideC = 0;
  bool b_kn = false;  // B stored [K][N] (N contiguous) instead of [N][K]
  bool a_km = false;  // A stored [K][M] (M contiguous, M a multiple of 8) instead of [M][K]
  int S = 1, H = 1;
  int nseg = 1;
  GemmSeg seg[3];
  // optional fp32 scratch for split-K partial tiles (decode-sized M); when
  // NULL or too small the kernels run without splitting K
  void *workspace = nullptr;
  size_t workspace_bytes = 0;
  // Row RMSNorm split over two products y = RMSNorm(x W1^T) W2^T (large-tile
  // kernel only; launch_gemm refuses them elsewhere).  Producer (x W1^T):
  // for output columns [0, rn_cols) (a multiple of 64) it writes, per row m
  // and 64-column chunk j, the sum of squares of the stored bf16 values to
  // rn_part[m * rn_cols / 64 + j], and stores those columns multiplied by
  // rn_gain (bf16).  Consumer (. W2^T, K = rn_cols): output row m is scaled
  // by 1 / sqrt(sum_j rs_part[m * rs_chunks + j] / (64 rs_chunks) + rs_eps),
  // j in order, before rounding.
  float *rn_part = nullptr;
  const void *rn_gain = nullptr;
  int rn_cols = 0;
  const float *rs_part = nullptr;
  int rs_chunks = 0;
  float rs_eps = 0.f;
  // RoPE of the stored values of column range rope_seg (large-tile kernel
  // only, and only where its tiles hold whole heads of that range; see
  // gemm_rope_fusable): in each dh-wide head, pair i of row m -- columns
  // (i, i + dh/2) for rope_conv 0 (half-split), (2i, 2i + 1) for 1
  // (interleaved) -- is rotated by rope_tab[m * dh + i] (cos) and
  // rope_tab[m * dh + dh/2 + i] (sin), as launch_rope's table holds them.
  const float *rope_tab = nullptr;
  int rope_seg = -1;
  int rope_conv = 0;
};

hipError_t launch_gemm(const GemmDesc &d, hipStream_t st);
// Whether launch_gemm runs a product of these sizes on the large-tile bf16
// kernel when both operands are K-contiguous (single batch, one column range
// starting at 0, ldb = K).
bool gemm_takes_large_tiles(int dtype, int M, int N, int K);
// Whether launch_gemm runs this product on the large-tile kernel.
bool gemm_uses_large_tiles(const GemmDesc &d);
// Whether launch_gemm can rotate column range `seg` of this product in its
// epilogue (bf16 large tiles whose columns hold whole heads of the range,
// heads a multiple of 16 wide, no split RMSNorm producer on the range).
bool gemm_rope_fusable(const GemmDesc &d, int seg);

// Scratch bytes launch_gemm can use for split-K partials of an M x N x K
// product (0 when it never splits).
size_t gemm_scratch_bytes(int dtype, int M, int N, int K, int batch);

// In-place RMSNorm of n columns of `rows` rows with pitch ld: x * (mean(x^2)
// + eps)^-1/2 * g, fp32 reduction.
hipError_t launch_rmsnorm(int dtype, void *x, int64_t rows, int64_t ld, int n,
                          const void *g, float eps, hipStream_t st);

// RoPE frequencies, resolved on the host in float64.
struct RopeTab {
  double inv_freq[64];
  float amp;        // multiplies cos and sin (YaRN mscale ratio)
  int pairs;        // rope_dim / 2
  int convention;   // 0 half-split, 1 interleaved
};

// In-place RoPE: element (t, h, i) at x + (t / S) * sb + (t % S) * ss + h * sh + i,
// position positions[t] (device) or t % S when positions is NULL.  With
// tab_out, token t's cos and sin (amplitude included) of its pairs are also
// written to tab_out[t * rope_dim + i] and tab_out[t * rope_dim + pairs + i]
// (the table a GEMM epilogue that rotates its output reads).
hipError_t launch_rope(int dtype, void *x, int64_t n_tok, int64_t S, int64_t sb,
                       int64_t ss, int n_heads, int64_t sh,
                       const int32_t *positions, const RopeTab &tab,
                       hipStream_t st, float *tab_out = nullptr);

// Copy `width` contiguous elements per row: dst row t at dst + t * ldd from
// src + t * lds (prefill latent output).
// Packed variable-length sequences (cu_seqlens [n_seq + 1], device): per
// token t its key range start[t] .. last[t] = t (its sequence's first token
// to itself), its position, and valid[t] = ok[0] = 1 for well-formed offsets
// (cu[0] = 0, non-decreasing, cu[n_seq] = total), else 0.
hipError_t launch_varlen_index(const int32_t *cu_seqlens, int n_seq, int64_t total, int32_t *start,
                               int32_t *last, int32_t *pos, int32_t *valid, int32_t *ok,
                               hipStream_t st);

// A chunk of q_len tokens per sequence against a latent cache (lens [B],
// device): lens_eff[b] = L_b when 0 <= L_b, L_b + q_len <= cap and all keys
// fit max_keys, else -1; kofs [B + 1] packed key offsets (sequence b's
// L_b + q_len keys start at kofs[b]); per query b * q_len + t its key range
// lo .. hi, position L_b + t and validity.
hipError_t launch_chunk_index(const int32_t *lens, int B, int q_len, int64_t cap, int64_t max_keys,
                              int32_t *lens_eff, int32_t *kofs, int32_t *lo, int32_t *hi, int32_t *pos,
                              int32_t *valid, hipStream_t st);
// Packed key stream of n_rows rows of width elements: row k is cache row
// k - kofs[b] of the sequence b that holds k, zeros from kofs[B] on.
hipError_t launch_gather_keys(int dtype, void *dst, int64_t n_rows, const void *cache, int64_t cap,
                              int width, const int32_t *kofs, int B, hipStream_t st);

// Block-scaled FP8 (E4M3 codes, E8M0 scale bytes stored [cols/128][ld_s], one
// per row): 1 x 128 activation tiles, 128 x 128 weight blocks (the block's
// byte repeated on each of its rows), and C = (A 2^sa)(B 2^sb)^T with A
// [M, K], B [N, K] bytes, scales padded to fp8_scale_pitch rows.
hipError_t launch_fp8_quant_rows(int dtype, const void *x, int64_t rows, int64_t cols, int64_t ldx, uint8_t *q,
                                 int64_t ldq, uint8_t *sexp, int64_t ld_s, hipStream_t st);
hipError_t launch_fp8_quant_blocks(int dtype, const void *w, int64_t rows, int64_t cols, int64_t ldw, uint8_t *q,
                                   int64_t ldq, uint8_t *sexp, int64_t ld_s, hipStream_t st);
hipError_t launch_fp8_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa, const uint8_t *b,
                           int64_t ldb, const uint8_t *sb, int64_t ld_sb, void *c, int c_dtype, int64_t ldc, int M,
                           int N, int K, hipStream_t st);
int64_t fp8_scale_pitch(int64_t rows);
// The same product (bf16 C) with the column-range output mapping of GemmSeg:
// B is one stacked code matrix with its scale bytes (seg[s].B and ldb
// unused); a channel-major range must start on a multiple of 256 columns.
struct Fp8GemmDesc {
  const uint8_t *a = nullptr, *sa = nullptr, *b = nullptr, *sb = nullptr;
  int64_t lda = 0, ld_sa = 0, ldb = 0, ld_sb = 0;
  int M = 0, N = 0, K = 0, S = 1, H = 1, nseg = 1;
  GemmSeg seg[3];
};
hipError_t launch_fp8_gemm_seg(const Fp8GemmDesc &d, hipStream_t st);

// Causal attention backward over BH heads of S rows: q, k [BH, S, dqk], v,
// o, dout [BH, S, dv] in, dq, dk [BH, S, dqk] and dvo [BH, S, dv] out (all of
// one dtype); lse and delta fp32 [BH * S] scratch, delta = lse + BH * S (the
// matrix-core kernels use the 2 BH S floats from lse as (lse, delta) pairs).
struct AttnBwdArgs {
  const void *q, *k, *v, *o, *dout;
  void *dq, *dk, *dvo;
  float *lse, *delta;
  int BH, S, dqk, dv;
  float scale;
};
hipError_t launch_attention_backward(int dtype, const AttnBwdArgs &a, hipStream_t st);
// The same on the matrix cores (bf16; d_qk, d_v one of 192/128, 96/64,
// 64/64); launch_attention_backward takes it where it applies.
bool attention_backward_mfma_supported(int dtype, int dqk, int dv);
hipError_t launch_attention_backward_mfma(const AttnBwdArgs &a, hipStream_t st);
// RMSNorm backward over rows of x [rows, n] (row pitches ldx, ldy, lddx):
// dx like x, dg fp32 [n] summed in a fixed order; scratch holds
// rmsnorm_backward_scratch_floats(rows, n) floats.
size_t rmsnorm_backward_scratch_floats(int64_t rows, int n);
hipError_t launch_rmsnorm_backward(int dtype, const void *x, int64_t ldx, const void *dy, int64_t ldy, const void *g,
                                   int64_t rows, int n, float eps, void *dx, int64_t lddx, float *dg, float *scratch,
                                   hipStream_t st);

// MLA backward layout helpers (16-byte chunks; widths and column offsets
// multiples of 8 elements):
//   to_heads = false: dst[(b S + s) dp + dcol + h w + c] = src[((b H + h) S + s) sp + scol + c]
//   to_heads = true:  dst[((b H + h) S + s) dp + dcol + c] = src[(b S + s) sp + scol + h w + c]
hipError_t launch_permute_heads(int dtype, bool to_heads, const void *src, int64_t sp, int scol, void *dst,
                                int64_t dp, int dcol, int w, int B, int S, int H, hipStream_t st);
// kh [B, H, S, dn + dr] = [k_nope [B, H, S, dn] ‖ shared k_pe (rows of pitch ld_kpe)]
hipError_t launch_build_keys(int dtype, const void *kn, const void *kpe, int64_t ld_kpe, void *kh, int dn, int dr,
                             int B, int S, int H, hipStream_t st);
// dst[(b S + s) ldd + c] = sum over h in order of src[((b H + h) S + s) sp + scol + c], c < w
hipError_t launch_head_sum(int dtype, const void *src, int64_t sp, int scol, void *dst, int64_t ldd, int w, int B,
                           int S, int H, hipStream_t st);
// dst[c ldd + r] = src[r lds + c] for r < R, c < C (bf16; R, C, lds, ldd
// multiples of 8, pointers 16-byte aligned)
hipError_t launch_transpose(const void *src, int64_t lds, int R, int C, void *dst, int64_t ldd, hipStream_t st);
// pos[t] = -(t % S)
hipError_t launch_neg_positions(int32_t *pos, int64_t n, int S, hipStream_t st);

hipError_t launch_copy_rows(int dtype, void *dst, int64_t ldd, const void *src,
                            int64_t lds, int64_t rows, int width,
                            hipStream_t st);

// Decode: write row t of src (width elements) into cache[b, lens[b]] when
// 0 <= lens[b] < cap.
// Write the q_len new latent rows of each sequence: token row b*q_len + t of
// src (pitch lds) goes to cache row lens[b] + t; a sequence with lens[b] < 0
// or lens[b] + q_len > cap is left untouched.
hipError_t launch_cache_append(int dtype, void *cache, int64_t cap,
                               const int32_t *lens, int q_len, const void *src,
                               int64_t lds, int64_t batch, int width,
                               hipStream_t st);

// pos[b*q_len + t] = lens[b] + t
hipError_t launch_decode_positions(const int32_t *lens, int batch, int q_len,
                                   int32_t *pos, hipStream_t st);

struct PrefillAttnArgs {
  const void *q;      // [B, H, S, dn + dr]
  const void *k_nope; // [B, H, S, dn]
  const void *k_pe;   // rows of pitch ld_kpe, token t = b * S + s
  int64_t ld_kpe;
  const void *vt;     // [B, H, dv, S]  (channel-major, keys contiguous)
  void *o;            // [B * S, H * dv]
  int B, S, H;
  float scale;
  // Key ranges (B = 1; packed sequences, chunks against a cache): query t
  // takes keys kv_lo[t] .. kv_hi[t] (inclusive, both non-decreasing in t) of
  // a key stream of Sk tokens (k_nope, k_pe and vt hold Sk keys instead of S);
  // valid[t] == 0 makes query t's output NaN.  kv_lo NULL: causal over S.
  const int32_t *kv_lo = nullptr;
  const int32_t *kv_hi = nullptr;
  const int32_t *valid = nullptr;
  int Sk = 0;
};

hipError_t launch_prefill_attention(int dtype, int dn, int dr, int dv,
                                    const PrefillAttnArgs &a, hipStream_t st);

// B sequences with q_len new tokens each; H = q_len * heads_per_tok query
// heads per sequence (token t's head h is query head t*heads_per_tok + h).
// Sequence b holds lens[b] + q_len cache rows; token t sees rows
// 0..lens[b] + t.
struct DecodeAttnArgs {
  const void *q_lat;  // [B, H, r + dr]  absorbed query ‖ post-RoPE q_pe
  const void *cache;  // [B, cap, r + dr]
  const int32_t *lens;
  void *o_lat;        // [B, H, r]
  void *part_o;       // [(n_blocks + B), ceil(H/32)] blocks of 32 heads x r padded to 32
                      // (MFMA accumulator order); bf16 for a bf16 cache, else fp32
  float *part_ml;     // [(n_blocks + B), H, 2]
  int64_t cap;
  int B, H;
  int q_len = 1, heads_per_tok = 0;
  int n_blocks;
  float scale;
};

hipError_t launch_decode_attention(int dtype, int r, int dr,
                                   const DecodeAttnArgs &a, hipStream_t st);
hipError_t launch_decode_merge(int dtype, int r, const DecodeAttnArgs &a,
                               hipStream_t st);

int decode_blocks(int q_len);

// q_lat[b, h, 0:r] = W_uk_h^T q_nope[b, h]: q_nope row b at qn + b*ldq + h*dn,
// W_uk rows h*dn + k of length r, q_lat row b head h at qlat + b*ldo +
// h*head_stride.  bf16 with dn = 128 only; anything else returns
// hipErrorInvalidValue (the caller falls back to the general GEMM).
hipError_t launch_absorb(int dtype, int dn, int r, int H, int B, const void *qn, int64_t ldq,
                         const void *wuk, void *qlat, int64_t ldo, int64_t head_stride,
                         hipStream_t st);

}  // namespace mla
