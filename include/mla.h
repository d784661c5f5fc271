/*
 * mla.h -- C ABI of the MLA decode library (libmla.so, AMD gfx950 / MI355X).
 *
 * One decode step of Multi-head Latent Attention over the compressed latent
 * KV cache, with W^UK absorbed into the query and W^UV applied after the
 * latent-space weighted sum.  Sources, cited by page title and section /
 * equation:
 *   "DeepSeek-V2: Strong, Economical, Efficient" -- section 2.1.2 (low-rank
 *     key-value joint compression; only c^KV is cached; W^UK can be absorbed
 *     into the query side and W^UV into the output side), section 2.1.3
 *     (decoupled RoPE: per-head q^R, one shared k^R per token, cached next to
 *     c^KV), Appendix C (full formulas; absorption by associativity of the
 *     matrix products), section 3.2.1 (n_h = 128, d_h = 128, d_c = 512,
 *     d_h^R = 64).
 *   "DeepSeek-V3 Technical Report" notes, MLA section -- the equations for
 *     k^C, k^R, v^C, q^C, q^R and the attention-output equation
 *     o_{t,i} = sum_{j<=t} softmax_j(q_{t,i}.k_{j,i} / sqrt(d_h + d_h^R)) v^C_{j,i}.
 *
 * With the absorbed query q~_{t,i} = [W^UK_i^T q^C_{t,i} ; q^R_{t,i}] and the
 * cache row K_j = [c^KV_j ; k^R_j] (d_c + d_h^R elements), the score is
 * q~.K_j / sqrt(d_h + d_h^R), the latent output is
 * latent_{t,i} = sum_j p_j c^KV_j, and o_{t,i} = W^UV_i latent_{t,i}.
 *
 * Conventions common to every call
 *   - All pointers are DEVICE pointers unless the name ends in _host.
 *   - All tensors are dense, row-major, and start 16-byte aligned.
 *   - The caller allocates and owns every buffer, including the workspace.
 *     The library allocates no memory and keeps no state between calls
 *     (except the device array of mla_decode_attn_noalloc, below).
 *   - Every call enqueues work on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns without synchronising.  Results are ready when the
 *     stream reaches that point.
 *   - Return value: MLA_OK (0) when the work was enqueued, else a negative
 *     mla_status_t.  All argument checks run on the host before any HIP call;
 *     on error nothing is enqueued and no buffer is touched.
 *   - Weights W^UK / W^UV are stored [n_h, d_h, d_c]: head i is the row block
 *     [i*d_h, (i+1)*d_h) of the d_h n_h x d_c matrix.
 *   - Query tokens are numbered n = b*T + tau (sequence b, query tau < T).
 *     A sequence of KV length L_b holds its T query tokens as its last T
 *     rows; query tau sits at position L_b - T + tau and attends to cache
 *     rows 0 .. L_b - T + tau (the sum includes the current token).
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_DIMS = -2,        /* dimension fields inconsistent or out of range */
  MLA_ERR_DTYPE = -3,       /* unknown or unsupported dtype combination */
  MLA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MLA_ERR_SEQLEN = -5,      /* some L_b < 1, L_b < T, or L_b beyond capacity */
  MLA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required */
  MLA_ERR_UNSUPPORTED = -7, /* valid request the library does not implement */
  MLA_ERR_LAUNCH = -8,      /* the HIP runtime rejected a kernel launch */
  MLA_ERR_ARG = -9          /* a count, size or flag argument is invalid */
} mla_status_t;

typedef enum mla_dtype {
  MLA_F32 = 0,      /* IEEE binary32 */
  MLA_BF16 = 1,     /* bfloat16 */
  MLA_FP8_E4M3 = 2, /* OCP FP8 E4M3 ("e4m3fn", max 448), KV cache only */
  MLA_FP6_E2M3 = 3  /* 6-bit cache (KV cache only, d_c + d_h^R = 576): OCP
                       microscaling FP6 E2M3 codes (max 7.5) with one E8M0
                       power of two per 32 elements, see mla_cache_append */
} mla_dtype_t;

/* Problem dimensions and number formats (a plain value struct). */
typedef struct mla_dims {
  int32_t n_heads;     /* n_h */
  int32_t d_head;      /* d_h   (per-head dim of q^C, k^C, v^C) */
  int32_t d_latent;    /* d_c   (KV compression dim) */
  int32_t d_rope;      /* d_h^R (decoupled RoPE dim, even) */
  int32_t page_size;   /* tokens per page of a paged cache; must be 64 */
  int32_t kv_dtype;    /* cache format: MLA_F32, MLA_BF16, MLA_FP8_E4M3 or
                          MLA_FP6_E2M3 */
  int32_t q_dtype;     /* format of queries, weights, q_abs and o:
                          MLA_F32 or MLA_BF16 */
  float softmax_scale; /* 0 -> 1/sqrt(d_head + d_rope) */
  float rope_base;     /* RoPE base; 0 -> 10000 */
  int32_t precision;   /* an mla_precision_t, see below */
  /* Context extension of the RoPE parts (YaRN, which "DeepSeek-V2",
   * section 3, long context extension, applies to the decoupled key and
   * query only: s = 40, alpha = 1, beta = 32, 4K training context).
   * yarn_factor <= 1 (or 0): plain RoPE.  Otherwise pair k's frequency
   * theta_k = base^(-2k/d_h^R) becomes
   *   (1 - g) theta_k / s + g theta_k,
   *   g = clamp((r_k - alpha) / (beta - alpha), 0, 1),
   *   r_k = yarn_orig_len * theta_k / (2 pi)   (turns over the old context),
   * in every rotation the library applies (mla_absorb_q, mla_cache_append,
   * mla_kv_produce), and when softmax_scale is 0 the attention scale is
   * (yarn_coef * ln s + 1)^2 / sqrt(d_h + d_h^R) (the pages' length scaling
   * factor sqrt(t) = c ln s + 1, taken as a factor t on every logit;
   * c = 0.0707 for DeepSeek-V2, 0.1 in the DeepSeek-V3 notes).  Zeroed
   * fields keep the plain behaviour.                                       */
  float yarn_factor;   /* s */
  float yarn_alpha;    /* alpha > 0 */
  float yarn_beta;     /* beta > alpha */
  int32_t yarn_orig_len; /* original context length L (tokens), >= 1 */
  float yarn_coef;     /* c >= 0 */
} mla_dims_t;

/* Arithmetic of the absorbed query and the attention (inputs and weights are
 * always read in q_dtype / kv_dtype).  bf16 rounding of the absorbed query
 * moves a score s by about 2^-9 of the query-key dot product, and rounding a
 * softmax weight to bf16 moves it by up to 2^-9 of itself: invisible when
 * the weights spread over many tokens, visible in the output when a few
 * cache rows of large norm take most of the weight.
 *   MLA_PREC_AUTO (default): the matrix-core kernels with bf16 operands.
 *     With n_heads a multiple of 128 and a BF16 cache, the absorbed query
 *     is stored as bf16 (hi, lo) pairs (hi = bf16(q), lo = bf16(q - hi)),
 *     the attention reads hi, and a work item whose largest scaled score
 *     exceeds 7 (natural-log units) is recomputed with split operands as in
 *     MLA_PREC_BF16X2.  Otherwise the same as MLA_PREC_BF16.
 *   MLA_PREC_FP32: the absorbed query is stored as fp32 whatever q_dtype
 *     is, and scores, weights and the weighted sum are formed in fp32 by
 *     the general (scalar) kernel.  Any dims.
 *   MLA_PREC_BF16: bf16 operands only (each softmax weight enters P.C
 *     rounded to 8 significant bits; the normaliser sums exactly the
 *     rounded weights).  Fastest; no recomputation.
 *   MLA_PREC_BF16X2: every work item on matrix cores with split operands:
 *     scores from the (hi, lo) query pair and weights as bf16 (hi, lo)
 *     pairs, i.e. relative errors of about 2^-17 instead of 2^-9; split
 *     partials in fp32.  Requires n_heads % 128 == 0 and a BF16 cache
 *     (MLA_ERR_UNSUPPORTED otherwise).                                      */
typedef enum mla_precision {
  MLA_PREC_AUTO = 0,
  MLA_PREC_FP32 = 1,
  MLA_PREC_BF16 = 2,
  MLA_PREC_BF16X2 = 3
} mla_precision_t;

/* Supported combinations:
 *   matrix-core path: d_h = 128, d_c = 512, d_h^R = 64, q_dtype = BF16
 *       (absorption and up-projection: any n_h; the absorption also with
 *       MLA_PREC_FP32); attention with precision AUTO, BF16 or BF16X2 and
 *         n_h % 32 == 0, (n_h*T) % 128 == 0, kv_dtype = BF16 or FP8_E4M3
 *           (blocks of 128 query rows: DeepSeek-V2 / V3, 128 heads; split
 *           operands in blocks of 64 rows, BF16 cache), or
 *         n_h % 16 == 0 otherwise, kv_dtype = BF16 or FP8_E4M3 (blocks of 16 or 32
 *           rows: e.g. DeepSeek-V2-Lite, 16 heads, T = 1..4);
 *       kv_dtype = FP6_E2M3: the 128-row blocks only (MLA_ERR_UNSUPPORTED
 *       for other shapes and for MLA_PREC_FP32 / MLA_PREC_BF16X2);
 *   general path: any n_h >= 1, d_h <= 256, d_c <= 512 (a multiple of 4),
 *       d_h^R <= 128 (even),
 *       every q_dtype / kv_dtype combination (e.g. the all-fp32 problems).
 * RoPE uses interleaved pairs (2k, 2k+1) rotated by pos * theta_k, theta_k =
 * base^(-2k/d_h^R) (or its YaRN form, above).
 */

/* ------------------------------------------------------------------------ */
/* Query absorption: "DeepSeek-V2", section 2.1.2 and Appendix C (W^UK is
 * absorbed into the query); decoupled RoPE of q^R, section 2.1.3.
 *
 *   q_abs[n, i, 0:d_c]        = W^UK_i^T q_nope[n, i, :]      (fp32 accumulate)
 *   q_abs[n, i, d_c:d_c+d_r]  = RoPE(q_rope[n, i, :], q_pos[n])   if q_pos
 *                             = q_rope[n, i, :]                   if q_pos NULL
 *
 * q_nope [n_tokens, n_h, d_h], q_rope [n_tokens, n_h, d_h^R],
 * w_uk [n_h, d_h, d_c]: q_dtype.  q_pos [n_tokens] int32 or NULL.
 * q_abs [n_tokens, n_h, d_c + d_h^R]: q_dtype (F32 when precision is
 * MLA_PREC_FP32), written (round to nearest); with q_dtype BF16, d_h = 128,
 * d_c = 512, d_h^R = 64, n_h % 128 == 0 and precision AUTO (BF16 cache) or
 * BF16X2 it is [n_tokens, n_h, 2, d_c + d_h^R] bf16: hi = bf16(q) then
 * lo = bf16(q - hi) of each row ("query pairs").
 * n_tokens >= 1.  Errors: MLA_ERR_UNSUPPORTED for BF16X2 on other shapes.  */
int32_t mla_absorb_q(const mla_dims_t* dims, const void* q_nope,
                     const void* q_rope, const void* w_uk,
                     const int32_t* q_pos, void* q_abs, int32_t n_tokens,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Cache append: writes cache rows [c^KV | k^R] of new tokens ("DeepSeek-V2",
 * section 2.1.3: c^KV and the shared, rotated k^R are the cached vectors;
 * "DeepSeek-V3 Technical Report" notes, MLA section, the boxed vectors).
 *
 * new_c [n_rows, d_c], new_kr [n_rows, d_h^R]: F32 when kv_dtype is F32,
 * else BF16.  Row r belongs to sequence seq_idx[r] at position pos[r]
 * (device int32 arrays of n_rows).  apply_rope != 0 rotates k^R at pos[r]
 * before it is stored.
 *
 * Layouts (D = d_c + d_h^R):
 *   contiguous (page_table == NULL): cache [B, max_len, D]; row =
 *       seq * max_len + pos.
 *   paged: cache [num_pages, page_size, D]; page_table [B, max_pages] int32;
 *       row = page_table[seq*max_pages + pos/page_size]*page_size
 *             + pos % page_size.
 * cache_rows is the capacity of the cache in rows (B*max_len or
 * num_pages*page_size).  A row whose target falls outside [0, cache_rows),
 * or whose position lies outside the sequence's pages, is skipped: the
 * kernel never writes outside the cache.
 *
 * kv_dtype FP8_E4M3: per row, s = amax|row| / 448 (float32, s = 1 if the row
 * is zero); each element stores the E4M3 code nearest to x / s (ties to
 * even, saturating at 448); kv_scale[row] = s.  kv_scale must be NULL for
 * other formats.
 *
 * kv_dtype FP6_E2M3 (the ~6-bit cache of "DeepSeek-V2", section 3.2.3,
 * training and inference efficiency, whose scheme the page leaves open):
 * each cache row is 452 bytes.  Elements are taken in blocks of 32 (18
 * blocks of the 576); block k has the shared exponent e_k = floor(log2
 * amax_k) - 2 kept in [-126, 127] (-126 for an all-zero block), so amax_k /
 * 2^e_k lies in [4, 8), and each element stores the E2M3 code nearest to
 * x / 2^e_k (ties to the even code, saturating at 7.5; sign = the sign bit
 * of x).  Bytes 24k .. 24k+23 hold block k's 32 codes, code i at bits
 * 6i .. 6i+5 of those bytes read as one little-endian integer; byte 432 + k
 * holds e_k + 127; bytes 450 and 451 are zero.  A stored element is
 * decode(code) * 2^e_k: 6.25 bits per element with the exponents.        */
int32_t mla_cache_append(const mla_dims_t* dims, const void* new_c,
                         const void* new_kr, const int32_t* seq_idx,
                         const int32_t* pos, const int32_t* page_table,
                         int32_t batch, int32_t max_pages, int32_t max_len,
                         int64_t cache_rows, int32_t apply_rope, void* cache,
                         float* kv_scale, int32_t n_rows, void* stream);

/* ------------------------------------------------------------------------ */
/* The decode step's two producers in one call: the query absorption of
 * mla_absorb_q ("DeepSeek-V2", section 2.1.2 and Appendix C; RoPE of q^R,
 * section 2.1.3) and the cache append of mla_cache_append (the cached c^KV
 * and k^R of section 2.1.3).  Arguments, layouts, results and errors are
 * those of the two calls (first the absorption's arguments, then the
 * append's); both are validated before anything is launched, and the
 * results are bit-identical to calling mla_absorb_q then mla_cache_append.
 * When both take their fast paths (d_h = 128, d_c = 512, d_h^R = 64,
 * q_dtype BF16, precision other than MLA_PREC_FP32, cache BF16, FP8_E4M3 or
 * FP6_E2M3) they run as one launch, since neither reads what the other
 * writes; otherwise as the two launches in that order.  q_abs must not
 * overlap the cache, its scales or the append's inputs.                   */
int32_t mla_absorb_append(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                          const void* w_uk, const int32_t* q_pos, void* q_abs,
                          int32_t n_tokens, const void* new_c, const void* new_kr,
                          const int32_t* seq_idx, const int32_t* pos,
                          const int32_t* page_table, int32_t batch, int32_t max_pages,
                          int32_t max_len, int64_t cache_rows, int32_t apply_rope,
                          void* cache, float* kv_scale, int32_t n_rows, void* stream);

/* ------------------------------------------------------------------------ */
/* Workspace of mla_decode_attn for the given host copy of the lengths and
 * split request (same planner as mla_decode_attn).  *bytes receives the
 * exact size: the split partials when some sequence is split, plus one
 * 4-byte flag per (work item, 128-row block) when precision AUTO may
 * recompute items with split operands; 0 when neither applies.            */
int32_t mla_decode_workspace_size(const mla_dims_t* dims,
                                  const int32_t* seq_lens_host, int32_t batch,
                                  int32_t q_tokens, int32_t num_splits,
                                  size_t* bytes);

/* ------------------------------------------------------------------------ */
/* Attention over the latent cache ("DeepSeek-V3 Technical Report" notes,
 * MLA section, attention-output equation, evaluated in absorbed form):
 *
 *   s_j = scale * q_abs[n, i, :] . cache_row_j        (j <= L_b - T + tau)
 *   out_latent[n, i, :] = sum_j softmax(s)_j * cache_row_j[0:d_c]
 *   out_lse[n, i]       = ln sum_j exp(s_j)
 *
 * q_abs as written by mla_absorb_q with the same dims ([B*T, n_h, D] in
 * q_dtype, F32 with MLA_PREC_FP32, or query pairs [B*T, n_h, 2, D]); cache
 * as in mla_cache_append (kv_scale for FP8 only).  seq_lens [B] int32 on the device; seq_lens_host: the same
 * values on the host (used to plan the split-KV work; they must agree).
 * num_splits = 0: the library splits long sequences into KV chunks to fill
 * the GPU; num_splits = S > 0: each sequence is cut into at most S chunks of
 * equal size (rounded up to 64 tokens).  Chunks are reduced with an LSE
 * combine.  workspace/ws_bytes: at least mla_decode_workspace_size() bytes
 * (may be NULL/0 when that size is 0).  out_latent [B*T, n_h, d_c] fp32,
 * out_lse [B*T, n_h] fp32.  Requires 1 <= T <= L_b for every b, and L_b <=
 * max_len (contiguous) or L_b <= max_pages*page_size (paged).             */
int32_t mla_decode_attn(const mla_dims_t* dims, const void* q_abs,
                        const void* cache, const float* kv_scale,
                        const int32_t* page_table, int32_t max_pages,
                        int32_t max_len, const int32_t* seq_lens,
                        const int32_t* seq_lens_host, int32_t batch,
                        int32_t q_tokens, int32_t num_splits, void* workspace,
                        size_t ws_bytes, float* out_latent, float* out_lse,
                        void* stream);

/* ------------------------------------------------------------------------ */
/* Allocation-free attention call, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Computes exactly what
 * mla_decode_attn computes, with the same kernels and the same split plan,
 * but the split-KV partials live in a device array of the library
 * (96 MiB per GPU, held from the first call on that GPU until the process
 * ends) instead of a caller workspace.  Arguments and errors are those of
 * mla_decode_attn without workspace / ws_bytes; a plan whose workspace
 * (mla_decode_workspace_size) exceeds 96 MiB returns MLA_ERR_WORKSPACE and
 * enqueues nothing.  The call itself allocates nothing.  All calls on one GPU
 * share its array: calls that overlap on one GPU (e.g. on two streams
 * without ordering between them) race and give undefined results.        */
int32_t mla_decode_attn_noalloc(const mla_dims_t* dims, const void* q_abs,
                                const void* cache, const float* kv_scale,
                                const int32_t* page_table, int32_t max_pages,
                                int32_t max_len, const int32_t* seq_lens,
                                const int32_t* seq_lens_host, int32_t batch,
                                int32_t q_tokens, int32_t num_splits,
                                float* out_latent, float* out_lse,
                                void* stream);

/* ------------------------------------------------------------------------ */
/* Value up-projection after the latent sum ("DeepSeek-V2", section 2.1.2 and
 * Appendix C: W^UV is applied to the latent output instead of forming
 * v^C for every cached token):
 *
 *   out[n, i, :] = W^UV_i latent[n, i, :]          (fp32 accumulate)
 *
 * latent [n_tokens, n_h, d_c] fp32; w_uv [n_h, d_h, d_c] q_dtype;
 * out [n_tokens, n_h, d_h] in out_dtype (MLA_F32, or MLA_BF16 rounded to
 * nearest).                                                               */
int32_t mla_up_proj_v(const mla_dims_t* dims, const float* latent,
                      const void* w_uv, void* out, int32_t out_dtype,
                      int32_t n_tokens, void* stream);

/* ------------------------------------------------------------------------ */
/* Latent-cache producer, fused with the append: the cached vectors of the
 * "DeepSeek-V3 Technical Report" notes, MLA section (c^KV_t = W^DKV h_t,
 * k^R_t = RoPE(W^KR h_t)), with the RMS norm that the "DeepSeek-V2" page
 * (section 3.2.1) places after the compressed latent vector:
 *
 *   c   = W^DKV h_t                       (fp32 accumulate)
 *   c_i = c_i g_i / sqrt(mean_j c_j^2 + norm_eps)     (when norm_gain != NULL)
 *   k   = W^KR h_t, rotated at position pos[t] when apply_rope
 *   cache row of (seq_idx[t], pos[t]) = [c | k], stored as mla_cache_append
 *   stores it (bf16 rounding, or a per-row fp8 scale and E4M3 codes).
 *
 * h [n_rows, d_model] in q_dtype; w_dkv_kr [d_c + d_h^R, d_model] in q_dtype,
 * rows 0..d_c-1 = W^DKV and rows d_c.. = W^KR (the order of the cache row);
 * norm_gain [d_c] fp32 or NULL; norm_eps >= 0.  seq_idx, pos, page_table,
 * batch, max_pages, max_len, cache_rows, apply_rope, cache, kv_scale, n_rows:
 * as mla_cache_append (rows whose slot falls outside the cache are skipped).
 * workspace/ws_bytes: at least mla_kv_produce_workspace_size() bytes (the
 * projection's fp32 partial sums over K blocks, or its fp32 rows when the
 * operands are fp32).  Errors: those
 * of mla_cache_append, MLA_ERR_ARG for d_model < 1 or a negative or
 * non-finite norm_eps, MLA_ERR_WORKSPACE; nothing is enqueued on an error.  */
int32_t mla_kv_produce_workspace_size(const mla_dims_t* dims, int32_t d_model,
                                      int32_t n_rows, size_t* bytes);
int32_t mla_kv_produce(const mla_dims_t* dims, const void* h, int32_t d_model,
                       const void* w_dkv_kr, const float* norm_gain,
                       float norm_eps, const int32_t* seq_idx,
                       const int32_t* pos, const int32_t* page_table,
                       int32_t batch, int32_t max_pages, int32_t max_len,
                       int64_t cache_rows, int32_t apply_rope, void* cache,
                       float* kv_scale, int32_t n_rows, void* workspace,
                       size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Attention output projection ("DeepSeek-V3 Technical Report" notes, MLA
 * section, the equation after the attention-output equation):
 *
 *   u[n, :] = W^O [o[n, 0, :]; o[n, 1, :]; ...; o[n, n_h-1, :]]  (fp32 accumulate)
 *
 * o [n_tokens, n_h, d_h] in o_dtype (MLA_F32 or MLA_BF16), e.g. written by
 * mla_up_proj_v; w_o [d_model, n_h*d_h] row-major in q_dtype; u [n_tokens,
 * d_model] in u_dtype (MLA_F32, or MLA_BF16 rounded to nearest even).
 * workspace/ws_bytes: at least mla_out_proj_workspace_size() bytes (fp32
 * partial sums; the size is 0, and workspace may be NULL, when the shapes do
 * not take the matrix-core path).  Errors: MLA_ERR_NULL, MLA_ERR_DTYPE,
 * MLA_ERR_ARG (d_model or n_tokens < 1), MLA_ERR_ALIGN (any pointer not
 * 16-byte aligned), MLA_ERR_WORKSPACE; nothing is enqueued on an error.   */
int32_t mla_out_proj_workspace_size(const mla_dims_t* dims, int32_t d_model,
                                    int32_t n_tokens, int32_t o_dtype,
                                    size_t* bytes);
int32_t mla_out_proj(const mla_dims_t* dims, const void* o, int32_t o_dtype,
                     const void* w_o, int32_t d_model, void* u, int32_t u_dtype,
                     int32_t n_tokens, void* workspace, size_t ws_bytes,
                     void* stream);

/* The output projection with W^O in a panel layout that the library writes
 * once (e.g. when the weights are loaded), so that each 32-row strip of
 * W^O streams from contiguous memory: element (f, k) of W^O [d_model, K]
 * (K = n_h*d_h) sits at element
 *     ((f / 32) * (K / 64) + k / 64) * 2048 + (f % 32) * 64 + k % 64
 * of w_packed, i.e. 32 x 64 panels of 4 KB, each strip of 32 rows stored as
 * its K/64 panels in order.  Same equation as mla_out_proj (the "DeepSeek-V3
 * Technical Report" notes, MLA section), and the same sums in the same order,
 * so its u is bit-identical to mla_out_proj's for the same inputs.
 *
 * mla_out_proj_pack: w_o [d_model, K] bf16 row-major -> w_packed (same size,
 * d_model*K*2 bytes, caller-owned, must not overlap w_o).
 * mla_out_proj_packed: o [n_tokens, n_h, d_h] bf16; w_packed as written by
 * mla_out_proj_pack; u [n_tokens, d_model] in u_dtype (MLA_F32 or MLA_BF16);
 * workspace/ws_bytes: at least mla_out_proj_workspace_size(dims, d_model,
 * n_tokens, MLA_BF16, ...) bytes.
 * Both need q_dtype = MLA_BF16 (else MLA_ERR_DTYPE), d_model % 32 == 0, K %
 * 256 == 0 and d_model*K*2 < 2^31 (else MLA_ERR_UNSUPPORTED).  Other errors:
 * MLA_ERR_NULL, MLA_ERR_ARG (d_model or n_tokens < 1, overlapping pack
 * buffers), MLA_ERR_ALIGN, MLA_ERR_WORKSPACE; nothing is enqueued on an
 * error.                                                                  */
int32_t mla_out_proj_pack(const mla_dims_t* dims, const void* w_o, int32_t d_model,
                          void* w_packed, void* stream);
int32_t mla_out_proj_packed(const mla_dims_t* dims, const void* o, const void* w_packed,
                            int32_t d_model, void* u, int32_t u_dtype, int32_t n_tokens,
                            void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Page-table range check (debug aid).  The cache rows of the "DeepSeek-V2"
 * page, section 2.1.3, are found through the page table of the paged layout
 * described at mla_cache_append; the attention and producer kernels do not
 * range-check the page ids they read (an id outside the cache is undefined
 * behaviour).  A caller that does not trust a table (debug builds, tables
 * built by other code) runs this check on the device first.
 *
 * page_table [batch, max_pages] int32 and seq_lens [batch] int32 (device).
 * For each sequence b the entries p < ceil(L_b / page_size) are checked to
 * lie in [0, n_pages); a length outside [0, max_pages * page_size] is
 * counted and the whole row is checked.  result (device int32[4], written by
 * the call; no clearing needed): [0] entries out of range, [1] flat index
 * b * max_pages + p of the first of them (-1 if none), [2] its value (0 if
 * none), [3] sequences with an out-of-range length.  One workgroup reads the
 * whole table: for debugging, not for the serving loop.
 * Errors: MLA_ERR_NULL, MLA_ERR_ARG (batch, max_pages or n_pages < 1, or
 * batch * max_pages > 2^31 - 1), dims errors as everywhere.               */
int32_t mla_check_page_table(const mla_dims_t* dims, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                             int64_t n_pages, int32_t* result, void* stream);

/* Static description of a status code (never NULL). */
const char* mla_status_string(int32_t status);

/* Library version as 10000*major + 100*minor + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
