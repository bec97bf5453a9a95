/*
 * mla.h — C ABI of the absorbed Multi-head Latent Attention (MLA) decode
 * library for AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [Mishra]   "Multi-head Latent Attention" (Neel Mishra).
 *   [Zhang]    "Multi-head latent attention" (zhangchitc.github.io).
 *   [LLMsBlog] "Multi-Head Latent Attention: How Low-Rank KV Compression
 *              Scales LLM Serving" (llms.blog).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" point to GPU memory owned by the caller; the
 *     library never allocates, frees or retains them past the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Entry points that take a stream are asynchronous: they enqueue work
 *     and return without synchronising the host.
 *   - Every argument check the host can make happens before any launch; a
 *     failed check launches nothing and returns a non-zero mla_status.
 *     The message is available from mla_last_error() on the same thread.
 *   - Device-side contents (block-table entries, sequence lengths) are not
 *     validated on the fast path; mla_decode_validate checks them.
 *   - All tensors are dense row-major with the shapes given; element types
 *     are given per argument. bf16 is the upper half of an IEEE binary32.
 *     fp8 is OCP e4m3fn (bias 7, max 448, no infinities).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, bad enum */
  MLA_ERR_UNSUPPORTED = 2,        /* valid but not built: dims/dtype combination */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,
  MLA_ERR_MISALIGNED = 4,         /* a device pointer is not 16-byte aligned */
  MLA_ERR_HIP = 5,                /* the HIP runtime reported an error */
  MLA_ERR_BAD_CONTENTS = 6        /* mla_decode_validate found a bad entry */
} mla_status;

typedef enum mla_dtype {
  MLA_FP32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2
} mla_dtype;

/* Tokens per cache page. The block table maps page k of a sequence (tokens
 * [64k, 64k+64)) to a physical page of the pool. */
#define MLA_PAGE_SIZE 64

/* Shape and type descriptor of one decode call (host memory, read only).
 *
 * The cached entry of a token is its latent c_j (d_c lanes) followed by its
 * rotated rope key k^R_j (d_rope lanes), one entry shared by all heads
 * ([Mishra] "Step 4: decoupled RoPE": the per-token cache is d_c + d_h^R;
 * [Zhang] "Decoupled RoPE": k^R is cached already rotated).
 */
typedef struct mla_decode_desc {
  int32_t batch;              /* B >= 1 sequences */
  int32_t q_len;              /* query tokens per sequence, >= 1; query m sits at
                                 position S_b - q_len + m and sees positions <= its own */
  int32_t n_heads;            /* n_h >= 1 */
  int32_t d_c;                /* latent width, multiple of 8, <= 1024 */
  int32_t d_rope;             /* rope width, multiple of 8, <= 256 */
  int32_t page_size;          /* must be MLA_PAGE_SIZE */
  int32_t max_blocks_per_seq; /* columns of block_table, >= 1 */
  int32_t cache_dtype;        /* MLA_FP32 | MLA_BF16 | MLA_FP8_E4M3 */
  int32_t q_dtype;            /* MLA_FP32 | MLA_BF16 (fp32 only with an fp32 cache) */
  int32_t out_dtype;          /* MLA_FP32 | MLA_BF16 */
  int32_t num_partitions;     /* 0 = automatic; else the number of equal ranges the
                                 batch's concatenated pages are cut into (split-KV) */
  int32_t plan_ready;         /* non-zero: the workspace already holds the plan that
                                 mla_decode_plan wrote for these seq_lens */
  int32_t flags;              /* 0, or MLA_DECODE_FP8_MATH */
} mla_decode_desc;

/* flags bit: with an FP8_E4M3 cache, d_c = 512, d_rope = 64 and bf16 queries
 * (the shapes the matrix-core kernel serves), compute the content scores on the fp8
 * matrix cores: the cached e4m3 codes are multiplied as stored against the
 * queries rounded to e4m3 (round to nearest even) after scaling each block of
 * 32 consecutive q_abs lanes by a power of two that puts its largest
 * magnitude in [128, 256); the rope part and the weighted sum stay in bf16
 * (the codes are widened exactly) with fp32 accumulation. This trades the
 * query's rounding to 3 mantissa bits for about half the matrix-core time of
 * the scores and no dequantisation pass. With any other cache type or shape
 * the flag has no effect. With it, batches above 256 sequences use the plan
 * kernel (one more launch) instead of forming the plan in the decode kernel. */
#define MLA_DECODE_FP8_MATH 1

/* Bytes of device workspace mla_decode needs for `d` (plan + split partials).
 * Pure host function; returns 0 if `d` is invalid (see mla_last_error). */
size_t mla_decode_workspace_size(const mla_decode_desc* d);

/* Writes the split plan (per-sequence page prefix sums) for device `seq_lens`
 * [B] int32 into `workspace` with one small kernel on `stream`; no host
 * synchronisation. A plan stays valid for any number of mla_decode calls
 * with plan_ready = 1 and the same seq_lens and desc (for example every
 * layer of one decode step). */
mla_status mla_decode_plan(const mla_decode_desc* d, const int32_t* seq_lens,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Absorbed-MLA decode attention in latent space.
 *
 * For sequence b, query m, head i, with S = seq_lens[b] and visible
 * positions j <= S - q_len + m:
 *   s_j  = scale * (q_abs[b,m,i,:] . c_j + q_rope[b,m,i,:] . k^R_j)
 *   a    = softmax(s)
 *   o_latent[b,m,i,:] = sum_j a_j c_j,   lse_out[b,m,i] = ln sum_j exp(s_j)
 * ([LLMsBlog] "Query Key Absorption": logits straight against the cached
 * latent plus the rope term; [Zhang] "Value absorption: weight and sum first,
 * project after": softmax weights sum the latents before any up-projection;
 * [Mishra] "Step 2: absorb the up-projections". scale is normally
 * 1/sqrt(d_h + d_R), the per-head content plus rope width.)
 * A query that sees no position gets o = 0 and lse = -inf.
 *
 * q_abs    device [B, q_len, n_h, d_c]     q_dtype
 * q_rope   device [B, q_len, n_h, d_rope]  q_dtype
 * cache    device page pool [n_pages, 64, row]:
 *            FP32/BF16: row = d_c + d_rope elements (c_j then k^R_j);
 *            FP8_E4M3:  row = d_c code bytes then d_rope bf16 (2*d_rope bytes);
 * cache_scale device [n_pages, 64] fp32 per-token scale s_j (FP8 only, else
 *            ignored): c_j = s_j * decode(code_j)
 * block_table device [B, max_blocks_per_seq] int32 physical page ids
 *            (entries past a sequence's last page are never read)
 * seq_lens device [B] int32, 0 <= S_b <= 64 * max_blocks_per_seq
 * o_latent device [B, q_len, n_h, d_c] out_dtype (written)
 * lse_out  device [B, q_len, n_h] fp32 natural-log sum-exp, or NULL
 * workspace device, >= mla_decode_workspace_size(d) bytes, 256-byte aligned;
 *            its contents are scratch except the plan (see plan_ready)
 * Calls that share a workspace must be ordered on one stream.
 */
mla_status mla_decode(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                      const void* cache, const float* cache_scale,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      void* o_latent, float* lse_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The two halves of mla_decode as separate calls, for callers that want the
 * split-KV kernel and the merge as two launches (to time them apart, or to run
 * other work on the stream between them). The partials stay in the
 * workspace in a layout private to the library, so only mla_decode_combine
 * can merge them, and only for the same desc, seq_lens and workspace.
 *
 * mla_decode_partial: the plan (unless plan_ready) and the split-KV kernel
 * only. It leaves, in the workspace, the partial output and log-sum-exp of
 * every (page range, sequence) piece (the matrix-core kernel leaves the
 * partial unnormalised, with its softmax row sum beside it); arguments as in
 * mla_decode. The workspace layout is private to the library.
 * mla_decode_combine: the log-sum-exp merge of those partials into
 * o_latent / lse_out (LSE = ln sum_r exp(lse_r), o = sum_r exp(lse_r - LSE) o_r),
 * exactly the softmax over all tokens ([Zhang] "Value absorption": one
 * softmax over every cached token weights the latents). Same desc and
 * workspace as the mla_decode_partial call it follows on the same stream. */
mla_status mla_decode_partial(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                              const void* cache, const float* cache_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float scale,
                              void* workspace, size_t workspace_bytes, void* stream);
mla_status mla_decode_combine(const mla_decode_desc* d, void* workspace, size_t workspace_bytes,
                              void* o_latent, float* lse_out, void* stream);

/* The same decode with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture that must not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation). Instead
 * of a caller-owned workspace it uses a fixed device array built into the
 * library: mla_decode_noalloc_max_workspace() bytes (72 MiB) on each GPU the
 * library runs on, held until the process ends. It allocates nothing and
 * calls no allocating routine. A call whose descriptor needs more than that
 * (mla_decode_workspace_size) returns MLA_ERR_WORKSPACE_TOO_SMALL before any
 * launch. The plan is formed on every call (plan_ready is ignored). Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads without ordering) race
 * and give wrong results; order them on one stream. Other arguments and
 * results as in mla_decode. */
mla_status mla_decode_noalloc(const mla_decode_desc* d, const void* q_abs, const void* q_rope,
                              const void* cache, const float* cache_scale,
                              const int32_t* block_table, const int32_t* seq_lens, float scale,
                              void* o_latent, float* lse_out, void* stream);
size_t mla_decode_noalloc_max_workspace(void);

/* Debug check of device contents (synchronises `stream`, copies to host):
 * every page id a sequence uses is in [0, n_pages), every length is in
 * [0, 64 * max_blocks_per_seq], and every non-empty sequence holds at least
 * q_len tokens (its own queries are cached before attention; mla_decode still
 * gives a query at a negative position o = 0 and lse = -inf). Returns
 * MLA_ERR_BAD_CONTENTS on the first violation, with its position in
 * mla_last_error(). */
mla_status mla_decode_validate(const mla_decode_desc* d, const int32_t* seq_lens,
                               const int32_t* block_table, int64_t n_pages, void* stream);

/* Offline key absorption ([Mishra] "Step 2", boxed identity; [LLMsBlog]
 * "Query Key Absorption"): W_qabs[i] = (W_UK_i)^T W_UQ_i.
 * W_UQ device fp32 [n_h*d_h, d_in], W_UK device fp32 [n_h*d_h, d_c]
 * (head i = rows [i*d_h, (i+1)*d_h)); W_qabs device fp32 [n_h, d_c, d_in]. */
mla_status mla_fold_query(const float* W_UQ, const float* W_UK, int32_t n_h, int32_t d_h,
                          int32_t d_c, int32_t d_in, float* W_qabs, void* stream);

/* Offline value absorption ([Mishra] "Step 2": out = (W^O W^UV) sum a c;
 * [Zhang] "Value absorption"): W_ov[:, i*d_c:(i+1)*d_c] = W_O[:, i*d_h:(i+1)*d_h] W_UV_i.
 * W_O device fp32 [d, n_h*d_h]; W_UV device fp32 [n_h*d_h, d_c];
 * W_ov device fp32 [d, n_h*d_c]. */
mla_status mla_fold_output(const float* W_O, const float* W_UV, int32_t n_h, int32_t d_h,
                           int32_t d_c, int32_t d, float* W_ov, void* stream);

typedef enum mla_proj_mode {
  MLA_PROJ_MERGED = 0,    /* out = W_ov concat_i(o_i) */
  MLA_PROJ_TWO_STAGE = 1  /* out = W_O concat_i(W_UV_i o_i): about 3.6x fewer
                             weight bytes at d_model 5120 ([Zhang] "Value
                             absorption", note on keeping the factors apart) */
} mla_proj_mode;

/* Latent-to-model output projection of T decoded rows.
 * o_latent device [T, n_h, d_c] (o_dtype MLA_FP32 | MLA_BF16);
 * MERGED:    W1 = W_ov fp32 [d, n_h*d_c], W2 unused;
 * TWO_STAGE: W1 = W_UV fp32 [n_h*d_h, d_c], W2 = W_O fp32 [d, n_h*d_h];
 * out device fp32 [T, d]. workspace: mla_output_proj_workspace_size bytes,
 * 256-byte aligned (TWO_STAGE: the fp32 head outputs W^UV_i o_i; both modes:
 * fp32 split-K partial tiles for few rows, summed in a fixed order). With
 * T up to 256 the products run on the fp32 matrix cores. */
size_t mla_output_proj_workspace_size(int32_t T, int32_t n_h, int32_t d_c, int32_t d_h, int32_t d,
                                      int32_t mode);
mla_status mla_output_proj(const void* o_latent, int32_t o_dtype, int32_t T, int32_t n_h,
                           int32_t d_c, int32_t d_h, int32_t d, int32_t mode,
                           const float* W1, const float* W2, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Cache write for T new tokens whose projections are given ([Zhang]
 * "Decoupled RoPE": k^R is cached already rotated).
 * rows device fp32 [T, d_c + d_rope]: the latent c_t, then the UNROTATED rope
 * key W^KR h_t; RoPE rotates interleaved pairs (2k, 2k+1) of the key by
 * pos * theta^(-2k/d_rope) (angle and sin/cos evaluated in fp64).
 * positions device int32 [T]; slots device int32 [T] = page*64 + offset of
 * each new row in the pool (negative: the token is skipped);
 * cache / cache_scale as in mla_decode for cache_dtype. FP8: per-token scale
 * s = amax/448 in fp32 over the d_c content lanes (1 if amax is 0) written to
 * cache_scale[slot]; codes are e4m3 of fp32(c / s), nearest-even, saturating. */
mla_status mla_cache_write(const float* rows, int32_t T, int32_t d_c, int32_t d_rope, float theta,
                           const int32_t* positions, const int32_t* slots, int32_t cache_dtype,
                           void* cache, float* cache_scale, void* stream);

/* Cache append from hidden states: c_t = W^DKV h_t ([Mishra] "Step 1: a
 * low-rank latent") and W^KR h_t, projected in fp32 into the workspace, then
 * mla_cache_write. h device fp32 [T, d]; W_DKV device fp32 [d_c, d];
 * W_KR device fp32 [d_rope, d]; workspace >= mla_cache_append_workspace_size
 * bytes, 256-byte aligned (the projected rows and split-K partial tiles). */
size_t mla_cache_append_workspace_size(int32_t T, int32_t d, int32_t d_c, int32_t d_rope);
mla_status mla_cache_append(const float* h, int32_t T, int32_t d, const float* W_DKV,
                            const float* W_KR, int32_t d_c, int32_t d_rope, float theta,
                            const int32_t* positions, const int32_t* slots,
                            int32_t cache_dtype, void* cache, float* cache_scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Absorbed query projection for T query tokens ([LLMsBlog] "Query Key
 * Absorption": q_abs_i = W_qabs_i x, formed once per step; "The Positional
 * Problem and Decoupled RoPE": q^R_i = RoPE(W^QR_i x, t)).
 * x device fp32 [T, d_in] (h_t, or the query latent c^Q_t);
 * W_qabs device fp32 [n_h, d_c, d_in]; W_QR device fp32 [n_h*d_rope, d_in];
 * positions device int32 [T]; q_abs out [T, n_h, d_c], q_rope out
 * [T, n_h, d_rope], both in q_dtype (MLA_FP32 | MLA_BF16); RoPE as in
 * mla_cache_write. workspace >= mla_absorb_query_workspace_size bytes,
 * 256-byte aligned. */
size_t mla_absorb_query_workspace_size(int32_t T, int32_t d_in, int32_t n_h, int32_t d_c,
                                       int32_t d_rope);
mla_status mla_absorb_query(const float* x, int32_t T, int32_t d_in, const float* W_qabs,
                            const float* W_QR, int32_t n_h, int32_t d_c, int32_t d_rope,
                            float theta, const int32_t* positions, int32_t q_dtype,
                            void* q_abs, void* q_rope, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---- prefill: the unabsorbed layer over whole prompts -------------------
 *
 * Processing all positions of a prompt at once is bound by arithmetic, and
 * there the layer keeps the unabsorbed form: the latent is expanded into
 * per-head keys and values ([LLMsBlog] opening section and "Hardware
 * Trade-offs and Tensor Parallelism"; [Mishra] "Step 2: absorb the
 * up-projections", last paragraph). Every product is bf16 on the matrix
 * cores with fp32 accumulation; intermediate activations are rounded to
 * bf16 between products. */

/* bf16 matrix-core GEMM, the building block of the prefill projections:
 * C[m, n] = sum_k A[m, k] B[n, k]. A device bf16 [M, K] (row stride lda),
 * B device bf16 [N, K] (row stride ldb: a weight stored [out, in]), C device
 * [M, N] (row stride ldc) in c_dtype (MLA_FP32 | MLA_BF16, rounded to nearest
 * even). K, lda and ldb must be multiples of 8 and A, B 16-byte aligned.
 * splits > 1 cuts K into that many pieces for skinny M (fp32 partial tiles in
 * `partial`, mla_gemm_bf16_partial_size bytes, summed in split order:
 * deterministic). */
mla_status mla_gemm_bf16(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda,
                         const void* B, int64_t ldb, void* C, int64_t ldc, int32_t c_dtype,
                         int32_t splits, float* partial, void* stream);
size_t mla_gemm_bf16_partial_size(int32_t M, int32_t N, int32_t K, int32_t splits);

typedef struct mla_prefill_desc {
  int32_t batch;        /* sequences, >= 1 */
  int32_t max_seq_len;  /* >= every sequence's length (sizes the launch grid) */
  int32_t d_model;      /* d: width of h and of the output */
  int32_t n_heads;      /* n_h */
  int32_t d_head;       /* d_h: per-head content query/key width = value width */
  int32_t d_rope;       /* d_R: rope width (shared key, per-head query) */
  int32_t d_c;          /* latent width */
  int32_t d_cq;         /* query latent width, or 0: queries projected from h */
  float rope_theta;     /* RoPE base (interleaved pairs, angle pos * theta^(-2k/d_R)) */
} mla_prefill_desc;

/* Weights of one layer, device bf16, each stored [out, in] row-major with
 * head i owning rows [i*width, (i+1)*width) of its block:
 *   W_DKVR [d_c + d_R, d]              W^DKV rows, then W^KR rows
 *   W_DQ   [d_cq, d] (NULL if d_cq = 0)
 *   W_UQR  [n_h*d_h + n_h*d_R, d_in]   W^UQ rows, then W^QR rows (d_in = d_cq or d)
 *   W_UKV  [2*n_h*d_h, d_c]            W^UK rows, then W^UV rows
 *   W_O    [d, n_h*d_h]                                                    */
typedef struct mla_prefill_weights {
  const void* W_DKVR;
  const void* W_DQ;
  const void* W_UQR;
  const void* W_UKV;
  const void* W_O;
} mla_prefill_weights;

/* Causal attention of the expanded form ([Zhang] "Value absorption": scores
 * (q^C_i . k^C_{j,i} + q^R_i . k^R_j) * scale, softmax over positions j <= t
 * of the same sequence, o = sum_j a_j v_{j,i}). Built for
 * (d_h, d_R) in {(128, 64), (64, 16), (64, 32), (128, 0)}.
 * Rows are tokens: T = cu_seqlens[batch] rows, sequence b = rows
 * [cu_seqlens[b], cu_seqlens[b+1]) (device int32 [batch + 1]).
 * q [T, ldq] bf16: head i's content query at columns [i*d_h, (i+1)*d_h);
 * q_rope [T, ldqr]: head i's rotated rope query at [i*d_R, (i+1)*d_R);
 * k [T, ldk]: head i's content key at [i*d_h, ...); k_rope [T, ldkr]: the
 * shared rotated rope key at [0, d_R); v [T, ldv]: head i's value at
 * [i*d_h, ...); o [T, ldo] bf16 output, head i at [i*d_h, ...); lse device
 * fp32 [n_h, T] (natural log of sum_j exp(score_j)) or NULL. scale > 0.
 * Row strides are multiples of 8 elements and inputs 16-byte aligned. */
mla_status mla_prefill_attention(const mla_prefill_desc* d, int64_t T, const void* q, int64_t ldq,
                                 const void* q_rope, int64_t ldqr, const void* k, int64_t ldk,
                                 const void* k_rope, int64_t ldkr, const void* v, int64_t ldv,
                                 const int32_t* cu_seqlens, float scale, void* o, int64_t ldo,
                                 float* lse, void* stream);

/* The whole unabsorbed layer for T prompt tokens (the steps are listed in
 * the source; [Mishra] "Step 1", "Step 4"; [Zhang] "The definitions",
 * "Decoupled RoPE", "Value absorption"):
 * h device bf16 [T, d]; cu_seqlens as above; positions device int32 [T]
 * (RoPE position of each token, normally its index in its sequence);
 * scale normally 1/sqrt(d_h + d_R); out device fp32 [T, d];
 * latent device fp32 [T, d_c + d_R] or NULL: the cached row of each token
 * (c_t, then k^R_t rotated), ready for mla_cache_write-style storage;
 * lse device fp32 [n_h, T] or NULL; workspace >= mla_prefill_workspace_size
 * bytes, 256-byte aligned. */
size_t mla_prefill_workspace_size(const mla_prefill_desc* d, int64_t T);
mla_status mla_prefill(const mla_prefill_desc* d, const void* h, int64_t T,
                       const int32_t* cu_seqlens, const int32_t* positions,
                       const mla_prefill_weights* w, float scale, float* out, float* latent,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Cached bytes per token and layer for a cache dtype: FP32 4*(d_c+d_rope);
 * BF16 2*(d_c+d_rope); FP8 d_c + 2*d_rope + 4 (codes, bf16 rope key, fp32
 * scale). With bf16, d_c 512 and d_rope 64 this is 2*576 bytes
 * ([Mishra] "Step 4": d_c + d_h^R numbers per token per layer). 0 if invalid. */
size_t mla_cache_bytes_per_token(int32_t d_c, int32_t d_rope, int32_t cache_dtype);

const char* mla_status_string(mla_status s);
/* Message of the last failed call on the calling thread ("" if none). */
const char* mla_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
