/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention forward.
 *
 * The operation is the DeepSeek-V3 MLA forward as the pages state it:
 *   "The Evolving Transformer -- DeepSeek V2 & V3", section 01 "Multi-head
 *   Latent Attention (MLA)": module MultiHeadLatentAttention (projections
 *   w_down_kv, w_up_k, w_up_v, w_kr, w_down_q, w_up_q, w_qr, wo; K = cat(K_nope,
 *   K_rope), Q = cat(Q_nope, Q_rope), V from the nope width; causal softmax
 *   attention scaled by 1/sqrt(dk); heads concatenated head-major; then wo) and
 *   the cache formula below it (c_kv is what gets cached).
 *   "DeepSeek-V3 Decoupled Implementation" README, "Architecture" list and
 *   "Key Dimensions (671B variant)" table: field names and V3 sizes, 512-dim
 *   latent, decoupled 64-dim RoPE stream, YaRN factor 40.
 *   "[DeepSeek-V3] Different rotary embedding implementation between
 *   DeepSeek-AI and Transformers": the two RoPE conventions.
 *
 * Where the pages are silent this library reads them as follows:
 *   - RMSNorm(c_q) = c_q * (mean(c_q^2) + eps)^-1/2 * q_norm, before both
 *     w_up_q and w_qr; there is no norm on c_kv unless the caller passes
 *     kv_norm gains (checkpoints that normalise the latent), in which case
 *     c_kv gets the same RMSNorm before it is cached or up-projected.
 *   - k_pe = w_kr x is ONE shared rope_dim vector per token (w_kr is
 *     [rope_dim, hidden]), broadcast to every head.
 *   - softmax scale = (nope + rope)^-1/2, times mscale(factor,
 *     mscale_all_dim)^2 under YaRN; the same scale in decode.
 *   - RoPE pair i turns by +pos * inv_freq_i, inv_freq_i = theta^(-2i/d),
 *     positions start at 0, angles are reduced in float64.
 *   - decode: the new token's position is cache_lens[b]; it attends to cache
 *     rows 0..cache_lens[b], itself included.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller allocates and owns every buffer.  The library never
 *     allocates device memory, never frees, and keeps no pointer past the call.
 *     Scratch comes from the caller's workspace, sized by *_workspace_size.
 *   - Asynchrony: work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *     null stream) and the call returns after the launches, with no host
 *     synchronisation.  Buffers must stay alive until the stream reaches the
 *     work.  Calls that run concurrently must not share a workspace.
 *   - Layout: row-major, C order.  Weights are nn.Linear matrices [out][in]
 *     (y = x W^T, no bias).  Every float tensor of one call has the dtype of
 *     cfg->dtype (fp32 or bf16); accumulation is always fp32.
 *   - Errors: arguments are validated before anything is launched; a failing
 *     call returns a status != MLA_OK, launches nothing, and leaves a message
 *     for mla_last_error().  The library never aborts the process.
 */
#ifndef MLA_MI355X_H
#define MLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MLA_API __attribute__((visibility("default")))
#else
#define MLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad size, bad enum value   */
  MLA_ERR_UNSUPPORTED = 2,        /* head-dim combination not instantiated    */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes below *_workspace_size   */
  MLA_ERR_HIP = 4                 /* a HIP launch failed (message has details)*/
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

typedef enum {
  /* pairs (i, i + d/2): the rotate-half ("Eleuther") formulation */
  MLA_ROPE_HALF_SPLIT = 0,
  /* pairs (2i, 2i + 1): the complex formulation of the DeepSeek-AI code;
   * the output keeps the interleaved layout */
  MLA_ROPE_INTERLEAVED = 1
} mla_rope_convention;

typedef struct {
  float theta;                    /* base, e.g. 10000                          */
  int32_t convention;             /* mla_rope_convention                       */
  float factor;                   /* YaRN scaling factor; 1 = plain RoPE       */
  int32_t original_max_position;  /* YaRN original context (4096 for V3)       */
  float beta_fast, beta_slow;     /* YaRN correction bounds (32, 1)            */
  float mscale, mscale_all_dim;   /* YaRN attention temperature terms (1, 1)   */
} mla_rope_params;

typedef struct {                  /* DeepSeek-V3 config field names            */
  int32_t hidden_size;            /* D   (7168 for V3)                         */
  int32_t num_heads;              /* H   (128)                                 */
  int32_t q_lora_rank;            /* r_q (1536)                                */
  int32_t kv_lora_rank;           /* r_kv (512)                                */
  int32_t qk_nope_head_dim;       /* d_n (128)                                 */
  int32_t qk_rope_head_dim;       /* d_r (64)                                  */
  int32_t v_head_dim;             /* d_v (128)                                 */
  float rms_norm_eps;             /* 1e-6                                      */
  float softmax_scale;            /* <= 0: default (see above)                 */
  mla_rope_params rope;
  int32_t dtype;                  /* mla_dtype of every float tensor           */
} mla_config;

typedef struct {                  /* device pointers, nn.Linear [out][in]      */
  const void *w_down_q;           /* [r_q, D]                                  */
  const void *q_norm;             /* [r_q]   RMSNorm gain                      */
  const void *w_up_q;             /* [H*d_n, r_q]                              */
  const void *w_qr;               /* [H*d_r, r_q]                              */
  const void *w_down_kv;          /* [r_kv, D]                                 */
  const void *kv_norm;            /* [r_kv] RMSNorm gain of c_kv, or NULL:     */
                                  /* NULL = no norm on c_kv (the pages name    */
                                  /* none); non-NULL: c_kv is RMS-normalised   */
                                  /* (eps = rms_norm_eps) with these gains     */
                                  /* before it is cached or up-projected       */
  const void *w_kr;               /* [d_r, D]   shared RoPE key              */
  const void *w_up_k;             /* [H*d_n, r_kv]                             */
  const void *w_up_v;             /* [H*d_v, r_kv]                             */
  const void *wo;                 /* [D, H*d_v]                                */
} mla_weights;

/* Byte offsets, inside the workspace, of the intermediates a prefill leaves
 * there (all in cfg->dtype unless stated, valid once the stream has run the
 * call):
 *   c_q   [B*S, r_q]           c_q = x w_down_q^T, then RMS-normalised in place
 *                              (q_rms_chunks = 0), or, with the RMSNorm split
 *                              over the down- and q up-projection (q_rms_chunks
 *                              > 0), c_q times the q_norm gains
 *   c_kv  [B*S, r_kv]          latent;  k_pe [B*S, d_r] post-RoPE
 *   q     [B, H, S, d_n+d_r]   q_nope ‖ post-RoPE q_pe per head
 *   k_nope[B, H, S, d_n]       v [B, H, d_v, S] (channel-major: keys contiguous)
 *   o     [B*S, H*d_v]         attention output, head-major columns
 *   q_rms_part [B*S, q_rms_chunks] fp32: per row, the sums of squares of c_q
 *                              over 64-column chunks; the normalised row is
 *                              c_q[r] * g / sqrt(sum / r_q + eps)
 * Row strides: c_q, c_kv and k_pe share one row of ld_down elements
 * (c_q at column 0, c_kv at r_q, k_pe at r_q + r_kv).  The split is used
 * for bf16 when r_q is a multiple of 64 and both products run on the
 * large-tile kernel (B*S >= 512, among others). */
typedef struct {
  size_t c_q, c_kv, k_pe, q, k_nope, v, o;
  int64_t ld_down;
  size_t q_rms_part;
  int64_t q_rms_chunks;
  size_t total;
} mla_prefill_layout;

/* ------------------------------------------------------------------ prefill
 * y = MLA(x) for x [B, S, D] at positions 0..S-1 with the causal mask.
 *   x          [B, S, D]             device, read
 *   y          [B, S, D]             device, written
 *   latent_out [B, S, r_kv + d_r]    device, written if not NULL: per token
 *              c_kv then the post-RoPE k_pe (the latent-cache row format)
 * Status: INVALID_ARGUMENT for NULL x/y/weights/workspace, B or S < 1, a
 * dimension < 1 or not a multiple of 8 (d_r: of 2, <= 128); UNSUPPORTED for a
 * (d_n, d_r, d_v) other than (16,8,16), (64,32,64), (128,64,128);
 * WORKSPACE_TOO_SMALL; HIP. */
MLA_API mla_status mla_prefill_workspace_size(const mla_config *cfg, int64_t batch,
                                      int64_t seq, size_t *bytes);
MLA_API mla_status mla_prefill_layout_of(const mla_config *cfg, int64_t batch,
                                 int64_t seq, mla_prefill_layout *layout);
MLA_API mla_status mla_prefill_forward(const mla_config *cfg, const mla_weights *w,
                               const void *x, int64_t batch, int64_t seq,
                               void *y, void *latent_out, void *workspace,
                               size_t workspace_bytes, void *hip_stream);

/* --------------------------------------------------- variable-length prefill
 * A batch of n_seq sequences of different lengths packed end to end: the
 * forward of each sequence on its own (the MLA section's causal mask within
 * the sequence, RoPE positions 0..len_b-1), run as one stream of
 * T = total_tokens rows so the projections see every token at once.
 *   cu_seqlens [n_seq + 1]         int32, device, read: sequence b is rows
 *              cu_seqlens[b] .. cu_seqlens[b+1]-1; a valid array starts at 0,
 *              never decreases (empty sequences are allowed) and ends at T
 *   x          [T, D]              device, read
 *   y          [T, D]              device, written
 *   latent_out [T, r_kv + d_r]     device, written if not NULL (as for
 *              mla_prefill_forward)
 * The offsets live in device memory, so the library checks them on the
 * device: for an invalid array every row of y is NaN (latent_out is still
 * written; rows use the clamped offsets).  The workspace holds the
 * intermediates of a B = 1, S = T prefill plus two int32 per token.
 * Status: as mla_prefill_forward, with T >= 1, 1 <= n_seq <= 2^24 and
 * cu_seqlens not NULL and 4-byte aligned. */
MLA_API mla_status mla_prefill_varlen_workspace_size(const mla_config *cfg, int64_t n_seq,
                                             int64_t total_tokens, size_t *bytes);
MLA_API mla_status mla_prefill_varlen_forward(const mla_config *cfg, const mla_weights *w,
                                      const void *x, const int32_t *cu_seqlens,
                                      int64_t n_seq, int64_t total_tokens, void *y,
                                      void *latent_out, void *workspace,
                                      size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------------- decode
 * One absorbed decode step (the cache formula of the MLA section, with
 * w_up_k folded into the query side and w_up_v into the output side, per
 * head, at run time):
 *   q_lat_h = w_up_k_h^T q_nope_h ; s_t = scale (q_lat_h . c_kv_t + q_pe_h . k_pe_t)
 *   o_lat_h = sum_t softmax(s)_t c_kv_t ; o_h = w_up_v_h o_lat_h ; y = wo o
 *   x            [B, D]                    device, one new token per sequence
 *   latent_cache [B, capacity, r_kv + d_r] device; rows [0, lens[b]) are read,
 *                row lens[b] is written with the new token's c_kv ‖ k_pe
 *   cache_lens   [B] int32                 device, read only (the caller
 *                advances it); 0 <= lens[b] < capacity is a device-side
 *                precondition: a sequence that violates it gets a NaN y row
 *                and no cache write.
 *   y            [B, D]                    device, written
 * Status: as prefill, except that the instantiated (kv_lora_rank, d_r) pairs
 * are (16,8), (128,32) and, in bf16 only, (512,64); also INVALID_ARGUMENT for
 * capacity < 1 or batch > 4096. */
typedef struct {
  size_t c_q, c_kv, q, q_lat, o_lat, o;   /* see mla_decode_layout_of */
  int64_t ld_down, n_splits, split_len;
  size_t total;
} mla_decode_layout;

MLA_API mla_status mla_decode_workspace_size(const mla_config *cfg, int64_t batch,
                                     int64_t cache_capacity, size_t *bytes);
MLA_API mla_status mla_decode_layout_of(const mla_config *cfg, int64_t batch,
                                int64_t cache_capacity,
                                mla_decode_layout *layout);
MLA_API mla_status mla_decode_absorbed(const mla_config *cfg, const mla_weights *w,
                               const void *x, int64_t batch,
                               void *latent_cache, int64_t cache_capacity,
                               const int32_t *cache_lens, void *y,
                               void *workspace, size_t workspace_bytes,
                               void *hip_stream);

/* Multi-token absorbed decode: q_len new tokens per sequence in one step
 * (the verification pass of speculative or multi-token decoding).  Token t
 * of sequence b sits at position lens[b] + t, its latent row is written at
 * cache row lens[b] + t, and it attends to rows 0..lens[b] + t: the cached
 * prefix and the new tokens up to itself (the causal tril mask of the MLA
 * section applied to the new tokens).  Per token the arithmetic is that of
 * mla_decode_absorbed, which is this call at q_len = 1.
 *   x            [B, q_len, D]            device
 *   latent_cache [B, capacity, r_kv + d_r] device; rows [0, lens[b]) read,
 *                rows lens[b] .. lens[b] + q_len - 1 written
 *   cache_lens   [B] int32                 device, read only (the caller
 *                advances it by q_len); 0 <= lens[b] and lens[b] + q_len <=
 *                capacity is a device-side precondition: a sequence that
 *                violates it gets NaN y rows and no cache write.
 *   y            [B, q_len, D]            device, written
 * With lens[b] = 0 and q_len = S this is the causal prefill of S tokens in
 * absorbed form, and in general a prefill chunk of q_len tokens against a
 * latent cache of lens[b] rows (the absorbed form costs 2(r_kv + d_r) + 2 r_kv
 * flops per query-row pair, against 2(d_n + d_r) + 2 d_v expanded, so it
 * suits short chunks).
 * Status: as mla_decode_absorbed; INVALID_ARGUMENT also for q_len outside
 * [1, 256] or above capacity.  The workspace depends on q_len: size it with
 * mla_decode_multi_workspace_size. */
MLA_API mla_status mla_decode_multi_workspace_size(const mla_config *cfg, int64_t batch,
                                           int64_t q_len, int64_t cache_capacity,
                                           size_t *bytes);
MLA_API mla_status mla_decode_absorbed_multi(const mla_config *cfg, const mla_weights *w,
                                     const void *x, int64_t batch, int64_t q_len,
                                     void *latent_cache, int64_t cache_capacity,
                                     const int32_t *cache_lens, void *y,
                                     void *workspace, size_t workspace_bytes,
                                     void *hip_stream);

/* Chunked prefill against a latent cache, expanded form: the same operation
 * as mla_decode_absorbed_multi (token t of sequence b at position
 * lens[b] + t, its latent row written at cache row lens[b] + t, attending
 * rows 0..lens[b] + t), computed the prefill way: the cache rows 0 ..
 * lens[b] + q_len - 1 of every sequence (the prefix and the new rows) are
 * packed into one key stream, up-projected with w_up_k / w_up_v to per-head
 * keys and values (the MLA section's K_i and V_i from c_kv, k_pe shared), and
 * each query runs the causal softmax over its own sequence's keys.  This
 * costs 2(d_n + d_r) + 2 d_v flops per query-key pair plus the up-projection
 * of every key row, so it suits long chunks.
 *   x            [B, q_len, D]            device
 *   latent_cache [B, capacity, r_kv + d_r] device; rows [0, lens[b]) read,
 *                rows lens[b] .. lens[b] + q_len - 1 written, then read
 *   cache_lens   [B] int32                 device, read only; a sequence with
 *                lens[b] < 0 or lens[b] + q_len > capacity gets NaN y rows
 *                and no cache write
 *   max_keys     host bound on the packed keys, sum over usable sequences of
 *                lens[b] + q_len: it sizes the workspace (per key: the latent
 *                row plus H (d_n + d_v) expanded elements, 64 KB at V3 sizes
 *                in bf16); when the keys exceed it every y row is NaN and no
 *                cache row is written
 *   y            [B, q_len, D]            device, written
 * Status: INVALID_ARGUMENT for NULL or misaligned pointers, B outside
 * [1, 4096], q_len outside [1, capacity], max_keys outside [q_len, 2^24],
 * B * q_len > 2^24, or a bad config; UNSUPPORTED, WORKSPACE_TOO_SMALL and HIP
 * as for mla_prefill_forward. */
MLA_API mla_status mla_prefill_chunk_workspace_size(const mla_config *cfg, int64_t batch,
                                            int64_t q_len, int64_t cache_capacity,
                                            int64_t max_keys, size_t *bytes);
MLA_API mla_status mla_prefill_chunk(const mla_config *cfg, const mla_weights *w, const void *x,
                             int64_t batch, int64_t q_len, void *latent_cache,
                             int64_t cache_capacity, const int32_t *cache_lens,
                             int64_t max_keys, void *y, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

/* --------------------------------------------------------------------- RoPE
 * In-place RoPE of x[t, h, 0..rope_dim) at positions[t] (device int32 [n_tokens]),
 * element (t, h, i) at x + t*token_stride + h*head_stride + i (strides in
 * elements).  Convention, theta and YaRN from *params (host struct).
 * Status: INVALID_ARGUMENT for NULL x/positions/params, n_tokens < 0,
 * n_heads < 1, rope_dim odd, < 2 or > 128, bad dtype or convention. */
MLA_API mla_status mla_rope_apply(void *x, int32_t dtype, int64_t n_tokens,
                          int32_t n_heads, int32_t rope_dim,
                          int64_t token_stride, int64_t head_stride,
                          const int32_t *positions,
                          const mla_rope_params *params, void *hip_stream);

/* ------------------------------------------------------------------- FP8
 * Block-scaled FP8 projection products, after the FP8 scheme of the "Deep
 * Seek V3" notes (section "infrastructure", the FP8 bullets): fine-grained
 * quantisation, tile-wise for activations and block-wise for weights, scales
 * from the maxima of each tile, E4M3 for every tensor, accumulation above FP8
 * precision.
 *
 * Codes are OCP E4M3 bytes (bias 7, largest finite 448).  A tile's scale is
 * the power of two 2^e, e the smallest with amax <= 448 * 2^e (e = 0 for an
 * all-zero tile, clamped to [-127, 127]); its codes are x / 2^e rounded to
 * nearest, ties to even.  Scales are stored as E8M0 bytes (value
 * 2^(byte - 127)) in k-block-major order: the byte of row r for columns
 * [128 kb, 128 kb + 128) sits at sexp[kb * ld_sexp + r], one byte per row
 * (a weight block's byte is repeated on each of its rows).  Non-finite
 * inputs give unspecified codes.  All pointers are device pointers; the
 * caller owns every buffer; the calls are asynchronous on hip_stream. */

/* Rows rounded up to a multiple of 256: the smallest ld_sa / ld_sb that
 * mla_fp8_gemm accepts for that many rows (returns -1 for rows < 0). */
MLA_API int64_t mla_fp8_scale_pitch(int64_t rows);

/* Activation tiles: 1 x 128 tiles of x [rows, cols] (dtype fp32 or bf16,
 * row pitch ldx elements) -> codes q [rows, cols] (row pitch ldq bytes) and
 * scale bytes sexp [cols / 128][ld_sexp].
 * Status: INVALID_ARGUMENT for NULL pointers (rows > 0), rows < 0, cols not
 * a positive multiple of 128, ldx < cols, ldq < cols, ldq odd, q not 2-byte
 * aligned, ld_sexp < rows, rows > 2^24, x not aligned to its element size or
 * a bad dtype. */
MLA_API mla_status mla_fp8_quantize_rows(const void *x, int32_t dtype, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *q, int64_t ldq, uint8_t *sexp,
                                 int64_t ld_sexp, void *hip_stream);

/* Weight blocks: 128 x 128 blocks of w [rows, cols] (rows = output
 * channels, cols = reduction; a partial last row block has its own scale)
 * -> codes q [rows, cols] and sexp [cols / 128][ld_sexp] (the block's byte on
 * each of its rows).
 * Status: INVALID_ARGUMENT as for mla_fp8_quantize_rows, except that ldq
 * must be a multiple of 16 and q 16-byte aligned. */
MLA_API mla_status mla_fp8_quantize_blocks(const void *w, int32_t dtype, int64_t rows, int64_t cols,
                                   int64_t ldw, uint8_t *q, int64_t ldq, uint8_t *sexp,
                                   int64_t ld_sexp, void *hip_stream);

/* C [M, N] = sum_k A[m, k] 2^(sa(m, k/128) - 127) B[n, k] 2^(sb(n, k/128) - 127),
 * fp32 accumulation, C written as c_dtype (fp32 or bf16) with row pitch ldc
 * elements.  a [M, K] and b [N, K] are E4M3 codes with row pitches lda and
 * ldb bytes (nn.Linear order: y = x W^T); sa [K / 128][ld_sa] and
 * sb [K / 128][ld_sb] are scale bytes as written by the quantisers.  Scale
 * rows past M (N) up to the pitch are read but never affect C.
 * Status: INVALID_ARGUMENT for NULL pointers (M > 0), M < 0, N < 1, M or N
 * above 2^24, K not a positive multiple of 128, lda or ldb below K or not a
 * multiple of 16, a or b not 16-byte aligned, ld_sa < mla_fp8_scale_pitch(M),
 * ld_sb < mla_fp8_scale_pitch(N), ld_sa / ld_sb not a multiple of 4, sa / sb
 * not 4-byte aligned, ldc < N, a bad c_dtype; for bf16 C also N or ldc not a
 * multiple of 8 or c not 16-byte aligned; for fp32 C, c not 4-byte aligned. */
MLA_API mla_status mla_fp8_gemm(const uint8_t *a, int64_t lda, const uint8_t *sa, int64_t ld_sa,
                        const uint8_t *b, int64_t ldb, const uint8_t *sb, int64_t ld_sb,
                        void *c, int32_t c_dtype, int64_t ldc, int64_t M, int64_t N, int64_t K,
                        void *hip_stream);

/* ------------------------------------------------------------- FP8 prefill
 * The prefill of mla_prefill_forward with its four projection products on
 * block-scaled FP8, the scheme of the "Deep Seek V3" notes (section
 * "infrastructure", the FP8 bullets): the linear layers run in E4M3 with
 * fine-grained scales (1 x 128 tiles of each activation, 128 x 128 blocks of
 * each weight, power-of-two scales as in mla_fp8_quantize_rows / _blocks)
 * and fp32 accumulation, while attention, RMSNorm and RoPE stay in higher
 * precision (bf16 storage, fp32 arithmetic).  The activations x, RMSNorm(c_q),
 * c_kv and the attention output o are quantised right after the kernel that
 * produces them.
 *
 * Weights: each projection's matrices are stacked by rows into one code
 * matrix (each matrix block-quantised on its own, so a block never spans
 * two matrices) with one scale byte per row and 128 columns. */
typedef struct {
  const uint8_t *codes;    /* [N, K] E4M3 codes, row pitch ld bytes          */
  int64_t ld;              /* >= K, multiple of 16                           */
  const uint8_t *scales;   /* [K / 128][ld_scales] E8M0 bytes, one per row    */
  int64_t ld_scales;       /* >= mla_fp8_scale_pitch(N), multiple of 4        */
} mla_fp8_matrix;

typedef struct {
  mla_fp8_matrix down;     /* [r_q + r_kv + d_r, D]: w_down_q, w_down_kv, w_kr */
  mla_fp8_matrix q_up;     /* [H (d_n + d_r), r_q]: w_up_q, then w_qr          */
  mla_fp8_matrix kv_up;    /* [H (d_n + d_v), r_kv]: w_up_k, then w_up_v       */
  mla_fp8_matrix out;      /* [D, H d_v]: wo                                   */
} mla_fp8_weights;

/* Bytes of the buffer mla_fp8_prepare_weights fills for *cfg.
 * Status: INVALID_ARGUMENT for a bad config; UNSUPPORTED unless bf16 with
 * hidden_size, q_lora_rank, kv_lora_rank and num_heads * v_head_dim multiples
 * of 128 and num_heads * qk_nope_head_dim a multiple of 256. */
MLA_API mla_status mla_fp8_weights_size(const mla_config *cfg, size_t *bytes);
/* Quantise the bf16 weights *w (device) into buffer (device, 256-byte
 * aligned, mla_fp8_weights_size bytes, owned by the caller) and describe the
 * result in *out (host struct; its pointers point into buffer).  Weights are
 * static: call once, reuse for every forward.  Asynchronous on hip_stream.
 * Status: as mla_fp8_weights_size; INVALID_ARGUMENT for NULL or misaligned
 * pointers; WORKSPACE_TOO_SMALL for a short buffer; HIP. */
MLA_API mla_status mla_fp8_prepare_weights(const mla_config *cfg, const mla_weights *w, void *buffer,
                                   size_t buffer_bytes, mla_fp8_weights *out, void *hip_stream);
MLA_API mla_status mla_prefill_fp8_workspace_size(const mla_config *cfg, int64_t batch, int64_t seq,
                                          size_t *bytes);
/* y = MLA(x) as mla_prefill_forward, with the projections on *w8.  From *w
 * only the RMSNorm gains are read (q_norm; kv_norm or NULL).  Arguments,
 * layouts, latent_out and stage events as mla_prefill_forward (stage 0 also
 * quantises x, stage 3 c_q and c_kv, stage 7 o).
 * Status: as mla_prefill_forward and mla_fp8_weights_size; INVALID_ARGUMENT
 * for NULL or misaligned FP8 matrices or pitches below their minimum. */
MLA_API mla_status mla_prefill_forward_fp8(const mla_config *cfg, const mla_weights *w,
                                   const mla_fp8_weights *w8, const void *x, int64_t batch,
                                   int64_t seq, void *y, void *latent_out, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------ attention backward
 * Gradients of the causal attention of "The Evolving Transformer -- DeepSeek
 * V2 & V3", section 01 (per head P = softmax(scale Q K^T, tril mask),
 * O = P V) for an upstream gradient dO:
 *   dV = P^T dO, dS = P * (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 *   dK = scale dS^T Q.
 * Rows are head-major and contiguous: q, k, dq, dk [batch_heads, seq, d_qk];
 * v, o, dout, dv [batch_heads, seq, d_v]; o is the forward output.  All
 * tensors have dtype (fp32 or bf16; arithmetic in fp32).  Device pointers,
 * 16-byte aligned, owned by the caller; the workspace holds 8 bytes per row
 * (the rows' log-sum-exp and rowsum(dO * O)).  Asynchronous on hip_stream.
 * Status: INVALID_ARGUMENT for NULL or misaligned pointers (rows > 0),
 * batch_heads or seq < 0, batch_heads * seq > 2^31 - 1, d_qk or d_v not a
 * multiple of 8 in [8, 256], a non-finite or non-positive scale or a bad
 * dtype; WORKSPACE_TOO_SMALL below the size; HIP for a failed launch. */
MLA_API mla_status mla_attention_backward_workspace_size(int64_t batch_heads, int64_t seq,
                                                 size_t *bytes);
MLA_API mla_status mla_attention_backward(int32_t dtype, int64_t batch_heads, int64_t seq,
                                  int32_t d_qk, int32_t d_v, float scale, const void *q,
                                  const void *k, const void *v, const void *o,
                                  const void *dout, void *dq, void *dk, void *dv,
                                  void *workspace, size_t workspace_bytes, void *hip_stream);

/* Allocation-free variant of mla_attention_backward, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight training or
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results
 * and errors as mla_attention_backward, without the workspace: the rows'
 * log-sum-exp and rowsum(dO * O) go to a scratch array built into the
 * library (8 bytes per row, 16 MB; each GPU the library runs on holds its own
 * copy until the process ends).  The call allocates nothing.  It runs on the
 * current device; a non-NULL hip_stream must belong to it.  Every call on a
 * GPU shares that GPU's scratch, which keeps the last call's contents (the
 * call writes every row it reads before reading it): calls that overlap on
 * one GPU, on any streams, race and give wrong results.
 * Status: as mla_attention_backward; INVALID_ARGUMENT also when
 * batch_heads * seq exceeds mla_attention_backward_noalloc_max_rows() or the
 * stream belongs to another device; HIP if the scratch cannot be located. */
MLA_API int64_t mla_attention_backward_noalloc_max_rows(void);
MLA_API mla_status mla_attention_backward_noalloc(int32_t dtype, int64_t batch_heads, int64_t seq,
                                          int32_t d_qk, int32_t d_v, float scale, const void *q,
                                          const void *k, const void *v, const void *o,
                                          const void *dout, void *dq, void *dk, void *dv,
                                          void *hip_stream);

/* RMSNorm backward (the norm on c_q of the MLA module of "The Evolving
 * Transformer -- DeepSeek V2 & V3", section 01; y = x r g with
 * r = (mean(x^2) + eps)^-1/2 per row): dx = r (g dy) - x r^3 mean(x g dy) and
 * dg = sum over rows of dy x r.  x, dy, dx [rows, n] contiguous and g [n] in
 * dtype (fp32 or bf16); dg fp32 [n] (summed over rows in order:
 * deterministic: fixed chunks of 64 rows, then the chunks in order); the
 * workspace holds mla_rmsnorm_backward_workspace_size bytes (4 per row plus
 * 4 per column per 64-row chunk).  Device pointers, 4-byte aligned, owned by
 * the caller.
 * Status: INVALID_ARGUMENT for NULL or misaligned pointers (rows > 0),
 * rows < 0 or > 2^31 - 1, n < 1 or > 2^20, eps < 0 or non-finite, a bad
 * dtype; WORKSPACE_TOO_SMALL below the workspace size; HIP for a failed
 * launch. */
MLA_API mla_status mla_rmsnorm_backward_workspace_size(int64_t rows, int32_t n, size_t *bytes);
MLA_API mla_status mla_rmsnorm_backward(int32_t dtype, const void *x, const void *dy, const void *g,
                                int64_t rows, int32_t n, float eps, void *dx, float *dg,
                                void *workspace, size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------------------ MLA backward
 * Every gradient of the prefill y = MLA(x) (the training half of the pages:
 * the forward of "The Evolving Transformer -- DeepSeek V2 & V3", section 01,
 * whose gradients the "DSV3 Native PyTorch Reference" README checks by
 * finite differences) for an upstream gradient dy: the chain rule back
 * through the output projection, the causal attention (per head, as
 * mla_attention_backward), the RoPE rotations (the rotation at negated
 * positions), the shared RoPE key (its gradient summed over heads in a fixed
 * order), the up-projections, the RMSNorms and the down-projections.  The
 * forward's intermediates are recomputed into the workspace first.
 *   x, dy      [B, S, D]   device, read
 *   dx         [B, S, D]   device, written
 *   grads      host struct of device pointers, written: each weight's
 *              gradient in cfg->dtype, shaped like the weight ([out][in]);
 *              the RMSNorm gains' gradients in fp32 (kv_norm only when
 *              w->kv_norm is not NULL; it may be NULL otherwise)
 * Weight gradients are sums over all B * S tokens.  Deterministic: every
 * sum runs in a fixed order.  Asynchronous on hip_stream; the caller owns
 * every buffer.
 * Status: as mla_prefill_forward; INVALID_ARGUMENT also for NULL or
 * misaligned dy, dx or gradients, or B * S * num_heads >= 2^31. */
typedef struct {
  void *w_down_q;                 /* [r_q, D]                                  */
  float *q_norm;                  /* [r_q]  fp32                               */
  void *w_up_q;                   /* [H*d_n, r_q]                              */
  void *w_qr;                     /* [H*d_r, r_q]                              */
  void *w_down_kv;                /* [r_kv, D]                                 */
  float *kv_norm;                 /* [r_kv] fp32, or NULL without kv_norm      */
  void *w_kr;                     /* [d_r, D]                                  */
  void *w_up_k;                   /* [H*d_n, r_kv]                             */
  void *w_up_v;                   /* [H*d_v, r_kv]                             */
  void *wo;                       /* [D, H*d_v]                                */
} mla_weight_grads;

MLA_API mla_status mla_backward_workspace_size(const mla_config *cfg, int64_t batch, int64_t seq,
                                       size_t *bytes);
MLA_API mla_status mla_backward(const mla_config *cfg, const mla_weights *w, const void *x,
                        int64_t batch, int64_t seq, const void *dy, void *dx,
                        const mla_weight_grads *grads, void *workspace, size_t workspace_bytes,
                        void *hip_stream);

/* ---------------------------------------------------------- measurement
 * While set, every mla_prefill_forward / mla_decode_absorbed call made on
 * this thread records events[k] (hipEvent_t handles the caller created) on
 * the call's stream just before it launches stage k, and events[n_stages]
 * after its last launch, for every index < n_events.  Stage order:
 *   prefill: 0 down projections, 1 RMSNorm, 2 k_pe RoPE (+ latent copy),
 *            3 q up-projection, 4 q_pe RoPE (no launch where the q
 *            up-projection rotates q_pe in its epilogue: bf16 on large
 *            tiles holding whole q_pe heads), 5 kv up-projection,
 *            6 attention, 7 output projection            (9 events)
 *   decode:  0 down projections, 1 RMSNorm, 2 k_pe RoPE + cache append,
 *            3 q up-projection, 4 q_pe RoPE, 5 absorption, 6 latent
 *            attention, 7 split merge, 8 un-absorption, 9 output projection
 *                                                         (11 events)
 * A NULL entry records nothing at that boundary (each recorded event costs
 * the stream a few microseconds, so a caller timing one stage may mark only
 * its ends).  events = NULL (or n_events = 0) switches it off.  The library keeps the
 * pointer array until then; the caller keeps it alive.  A failing
 * hipEventRecord makes the call return MLA_ERR_HIP. */
MLA_API mla_status mla_set_stage_events(void *const *events, int32_t n_events);

/* Softmax scale the library uses for *cfg (resolves softmax_scale <= 0). */
MLA_API float mla_softmax_scale(const mla_config *cfg);

/* Message of the last failing call on this thread ("" if none). */
MLA_API const char *mla_last_error(void);
MLA_API const char *mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_MI355X_H */
