/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The path has three stages, each an entry point below:
 *   1. lightning indexer: I[t,s] = sum_j w[t,j] * ReLU(q^I[t,j,:] . k^I[s,:]) over the
 *      preceding tokens s of the query's sequence;
 *   2. fine-grained token selection: the top-k positions of each score row;
 *   3. MLA in MQA mode over only the selected entries: every query head attends to
 *      the same latent cache entries (latent || RoPE key), values are the latent part.
 * Sources, by page title and section:
 *   "DeepSeek-V3.2 技术报告摘要" (summary of the V3.2 technical report), section 1,
 *     "关键设计：DeepSeek Sparse Attention (DSA)": ① Lightning Indexer (the formula,
 *     FP8 support), ② Fine-grained Token Selection, and the paragraph on the MLA-based
 *     implementation (MQA mode, one latent entry shared by all query heads);
 *   "DeepSeek-V3.2 -- Model techniques map", table "Checked in its code", rows
 *     "Indexer-selected sparse attention" (k = min(index_topk, row length), int32
 *     indices [B,S,topk]), "Multi-head latent attention" (entry = 512 latent + 64
 *     RoPE), "Partial RoPE" (192-d q/k head), "Learnable attention sink" and "Gated
 *     attention output" (both absent);
 *   "DeepSeek-V3.2" (model docs), section 1 "Model Introduction" (64 indexer heads x
 *     128, index_topk 2048, 128 heads) and section 5.3 "Rollout & SGLang" (bf16 cache,
 *     page size 64);
 *   "DeepSeek-V3.2-Exp" README, section "开源内核" (open kernels): an indexer-logits
 *     kernel with a paged version, separate from the sparse attention kernel.
 *
 * Conventions for every entry point
 *   - Tensors are row-major, contiguous, in device memory unless marked "host".
 *   - The caller owns every buffer, workspace included (sized by the *_workspace_size
 *     queries).  The library allocates nothing, keeps no state between calls and
 *     holds no pointer after it returns.  The dsa_rows struct is read on the host
 *     during the call only.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream) and the call returns after launch: inputs must stay alive until the
 *     stream has passed the work.  No host synchronisation, no device-to-host read,
 *     so a sequence of calls can be captured into a HIP graph.
 *   - Errors: the return value is a dsa_status; 0 is success.  All argument checks
 *     run on the host before anything is enqueued, so on an error nothing is
 *     launched.  A failed launch returns DSA_ERR_HIP.  Device-side contract breaches
 *     (a row_len beyond the cache, a page id out of range, a row_seq beyond num_seqs)
 *     are not checked and give undefined results.
 *   - num_rows == 0 is a valid empty call: DSA_OK, nothing launched.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2
#define DSA_PAGE_SIZE 64     /* tokens per cache page in the paged layout */
#define DSA_MAX_TOPK 2048    /* largest supported k (index_topk of the model) */
/* scratch of dsa_sparse_attention_decode_noalloc, held per GPU for the process's lifetime */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent layout */
    DSA_ERR_UNSUPPORTED = 2,   /* valid request the library has no kernel for */
    DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
    DSA_ERR_HIP = 4            /* a HIP launch failed */
} dsa_status;

typedef enum {
    DSA_F32 = 0,               /* IEEE binary32 */
    DSA_BF16 = 1,              /* bfloat16 */
    DSA_FP8_E4M3 = 2           /* OCP FP8 E4M3FN codes plus fp32 scales */
} dsa_dtype;

/* A ragged batch of query rows.  Query row r belongs to sequence row_seq[r] and sees
 * that sequence's positions 0 .. row_len[r]-1 (causal, its own token included: a
 * decode row has row_len = context length, prefill row t of a sequence has t+1).
 * The cache layout is either contiguous or paged:
 *   contiguous: position s of sequence b is cache row seq_start[b] + s;
 *   paged:      it is row page_table[b*max_pages + s/64]*64 + s%64 of a [pages,64,..]
 *               cache (64-token pages reached through a per-sequence page table). */
typedef struct dsa_rows {
    int32_t        num_rows;     /* host: R >= 0 */
    int32_t        num_seqs;     /* host: B >= 1 */
    const int32_t *row_seq;      /* [R] sequence of each row, in [0, B) */
    const int32_t *row_len;      /* [R] visible length, 1 <= row_len[r] <= max_row_len */
    int32_t        max_row_len;  /* host: >= every row_len; sizes grids, bounds ld */
    const int64_t *seq_start;    /* [B] contiguous layout, NULL for paged */
    const int32_t *page_table;   /* [B, max_pages] paged layout, NULL for contiguous */
    int32_t        max_pages;    /* host: paged only, >= ceil(max_row_len / 64) */
    int32_t        page_size;    /* host: paged only, must be DSA_PAGE_SIZE */
} dsa_rows;

/* Human-readable name of a status code (static storage). */
const char *dsa_status_string(int status);
/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

/* ---------------------------------------------------------------------------------
 * Stage 1: lightning-indexer scores ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ①).
 *   logits[r, s] = sum_{j<H} w[r,j] * ReLU(q[r,j,:] . k[cache row of s,:])  for s < row_len[r]
 * q       [R, H, D]  in `dtype` (f32, bf16, or e4m3 codes)
 * q_scale [R, H] f32 dequantisation scale of q (fp8 only, else NULL): q = code * q_scale
 * k       contiguous: [cache rows, D]; paged: [pages, 64, D]  in `dtype`
 * k_scale contiguous: [cache rows]; paged: [pages, 64]  f32 (fp8 only, else NULL)
 * w       [R, H] f32 head weights
 * logits  [R, ld_logits] f32 output; entries s >= row_len[r] are not written.
 * Supported: f32 with 1 <= H <= 64, 1 <= D <= 256; bf16 and fp8 with (H, D) = (64, 128).
 * dsa_indexer_logits needs rows->seq_start, dsa_indexer_logits_paged rows->page_table. */
int dsa_indexer_logits(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                       const void *q, const float *q_scale,
                       const void *k, const float *k_scale,
                       const float *w, float *logits, int64_t ld_logits, void *stream);
int dsa_indexer_logits_paged(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                             const void *q, const float *q_scale,
                             const void *k, const float *k_scale,
                             const float *w, float *logits, int64_t ld_logits, void *stream);

/* ---------------------------------------------------------------------------------
 * Stage 2: top-k token selection ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ②;
 * "Model techniques map", "Indexer-selected sparse attention": k capped at the row
 * length, int32 indices).
 * For each row r with n = row_len[r] valid scores logits[r, 0..n): the k_eff = min(k, n)
 * positions with the largest scores, ties broken toward the lower position, -0 == +0.
 * idx [R, k] int32 output: the selected positions in ascending order, then -1 padding.
 * Scores must be finite (NaN and infinities are not supported).  1 <= k <= 2048.
 * ws / ws_bytes: device scratch of at least dsa_topk_workspace_size(R, max_row_len, k)
 * bytes (may be NULL when that is 0); its contents need no initialisation.  Calls that
 * share one workspace must not run concurrently. */
size_t dsa_topk_workspace_size(int num_rows, int max_row_len, int k);
int dsa_topk(const float *logits, int64_t ld_logits, const int32_t *row_len, int num_rows,
             int max_row_len, int k, int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Stages 1 and 2 in one call: exactly the logits of dsa_indexer_logits(_paged) and the
 * indices of dsa_topk on them, for the same arguments.  For batches of few long rows (the
 * decode shape) the indexer workgroups also count their scores by the leading radix digit
 * of the selection as they produce them, so the selection starts from those counts instead
 * of a separate pass over the scores.
 * topk: k of dsa_topk;  idx [R, topk] int32 output as dsa_topk.
 * ws / ws_bytes: device scratch of at least dsa_indexer_topk_workspace_size(R,
 * max_row_len, dtype, topk) bytes (may be NULL when that is 0); needs no initialisation;
 * calls that share one workspace must not run concurrently.
 * Errors: those of dsa_indexer_logits and of dsa_topk. */
size_t dsa_indexer_topk_workspace_size(int num_rows, int max_row_len, int dtype, int k);
int dsa_indexer_topk(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                     const void *q, const float *q_scale, const void *k, const float *k_scale,
                     const float *w, float *logits, int64_t ld_logits, int topk, int32_t *idx,
                     void *ws, size_t ws_bytes, void *stream);
int dsa_indexer_topk_paged(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                           const void *q, const float *q_scale, const void *k,
                           const float *k_scale, const float *w, float *logits,
                           int64_t ld_logits, int topk, int32_t *idx, void *ws,
                           size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Stage 3: MLA in MQA mode over the selected entries ("DeepSeek-V3.2 技术报告摘要",
 * section 1, MLA-based implementation; "Model techniques map", "Multi-head latent
 * attention", "Learnable attention sink", "Gated attention output").
 * For row r, head h, and the valid entries s of idx[r,:] (0 <= s < row_len[r];
 * negative or larger entries are skipped):
 *   z_s = softmax_scale * q[r,h,:] . C[s,:]          (C = the d_qk-wide cache entry)
 *   out[r,h,:] = sum_s softmax(z)_s * C[s, 0:d_v]    (values = first d_v dims)
 *   lse[r,h]   = ln sum_s exp(z_s)
 * A row with no valid entry gets out = 0 and lse = -inf.  No sink, no gate.
 * q   [R, H, d_qk] in `dtype`;  kv contiguous [cache rows, d_qk] / paged [pages, 64, d_qk]
 * idx [R, k] int32 positions (e.g. from dsa_topk);  out [R, H, d_v] in `dtype`
 * lse [R, H] f32 natural-log sum-exp, or NULL.
 * softmax_scale must be finite and positive (DSA_ERR_INVALID_ARG otherwise).
 * Supported: f32 with 1 <= H <= 128, d_v <= d_qk <= 256;
 *            bf16 with H = 128, d_qk = 576, d_v = 512.  1 <= k <= 2048.
 * The decode entry points split the selections over several workgroups for few-row
 * batches and need ws of dsa_sparse_mla_workspace_size(R, H, d_v, k) bytes;
 * dsa_sparse_mla_prefill(_paged) never splits and takes ws = NULL, ws_bytes = 0. */
size_t dsa_sparse_mla_workspace_size(int num_rows, int n_heads, int d_v, int k);
int dsa_sparse_mla_decode(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                          float softmax_scale, const void *q, const void *kv,
                          const int32_t *idx, int k, void *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream);
int dsa_sparse_mla_decode_paged(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                                float softmax_scale, const void *q, const void *kv,
                                const int32_t *idx, int k, void *out, float *lse,
                                void *ws, size_t ws_bytes, void *stream);
int dsa_sparse_mla_prefill(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                           float softmax_scale, const void *q, const void *kv,
                           const int32_t *idx, int k, void *out, float *lse,
                           void *ws, size_t ws_bytes, void *stream);
/* Prefill (or a chunk of prefill over a cached prefix) on the 64-token paged cache
 * ("DeepSeek-V3.2" model docs, section 5.3: bf16 cache, page size 64). */
int dsa_sparse_mla_prefill_paged(const dsa_rows *rows, int dtype, int n_heads, int d_qk,
                                 int d_v, float softmax_scale, const void *q, const void *kv,
                                 const int32_t *idx, int k, void *out, float *lse,
                                 void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Stages 1-3 of a decode batch in one call ("DeepSeek-V3.2 技术报告摘要", section 1: the
 * indexer, the fine-grained selection and MLA in MQA mode over the selected entries):
 * exactly the logits and idx of dsa_indexer_topk(_paged) with (idx_dtype, idx_heads, idx_dim,
 * q_idx, q_idx_scale, k_idx, k_idx_scale, w, topk), and the out / lse of
 * dsa_sparse_mla_decode(_paged) with (dtype, n_heads, d_qk, d_v, softmax_scale, q, kv) on
 * those idx, bit for bit.  For batches of few long rows with the bf16 attention the last step
 * of the selection runs inside the attention workgroups (each split of a row selects the row's
 * positions from the survivors of the chunked selection, keeps its own slots and writes them
 * to idx), so the attention does not wait for a separate selection launch.
 * Arguments, layouts and their limits are those of the two calls; topk is also the attention's k.
 * ws / ws_bytes: device scratch of at least dsa_sparse_attention_decode_workspace_size(R,
 * max_row_len, idx_dtype, topk, n_heads, d_v) bytes (may be NULL when that is 0); needs no
 * initialisation; calls that share one workspace must not run concurrently.
 * Errors: those of the two calls (DSA_ERR_UNSUPPORTED for an fp8 attention). */
size_t dsa_sparse_attention_decode_workspace_size(int num_rows, int max_row_len, int idx_dtype,
                                                  int topk, int n_heads, int d_v);
int dsa_sparse_attention_decode(const dsa_rows *rows, int idx_dtype, int idx_heads, int idx_dim,
                                const void *q_idx, const float *q_idx_scale, const void *k_idx,
                                const float *k_idx_scale, const float *w, float *logits,
                                int64_t ld_logits, int topk, int32_t *idx, int dtype, int n_heads,
                                int d_qk, int d_v, float softmax_scale, const void *q,
                                const void *kv, void *out, float *lse, void *ws, size_t ws_bytes,
                                void *stream);
int dsa_sparse_attention_decode_paged(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                      int idx_dim, const void *q_idx, const float *q_idx_scale,
                                      const void *k_idx, const float *k_idx_scale, const float *w,
                                      float *logits, int64_t ld_logits, int topk, int32_t *idx,
                                      int dtype, int n_heads, int d_qk, int d_v,
                                      float softmax_scale, const void *q, const void *kv,
                                      void *out, float *lse, void *ws, size_t ws_bytes,
                                      void *stream);

/* dsa_sparse_attention_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same call
 * on the contiguous layout, with the same results bit for bit, but without a workspace
 * argument.  Its scratch is a static device array of DSA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; the call allocates nothing
 * (its first call on a device looks the array's address up).  Every call on one GPU uses
 * that GPU's one array, so calls that overlap on a GPU (other streams, other host threads)
 * race and must be serialised by the caller.  The scratch needs no initialisation.
 * Errors: those of dsa_sparse_attention_decode, and DSA_ERR_WORKSPACE when
 * dsa_sparse_attention_decode_workspace_size of the batch exceeds DSA_NOALLOC_SCRATCH_BYTES
 * (nothing is enqueued then). */
int dsa_sparse_attention_decode_noalloc(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                        int idx_dim, const void *q_idx, const float *q_idx_scale,
                                        const void *k_idx, const float *k_idx_scale,
                                        const float *w, float *logits, int64_t ld_logits, int topk,
                                        int32_t *idx, int dtype, int n_heads, int d_qk, int d_v,
                                        float softmax_scale, const void *q, const void *kv,
                                        void *out, float *lse, void *stream);

/* ---------------------------------------------------------------------------------
 * Masked MHA mode for short prefill ("DeepSeek-V3.2 技术报告摘要", section 1, "短序列优化":
 * short prefill runs DSA as masked MHA; "DeepSeek-V3.2 -- Model techniques map",
 * "Multi-head latent attention": 128 nope + 64 rope query/key dims, 128 value dims per head).
 * The latent entries the batch reaches ([c (512) | kr (64)], the layout of the MLA calls: for
 * each sequence, its positions below the longest row_len of its rows) are first decompressed
 * per head h: K[s,h] = [W_UK[h] c_s | kr_s] (192 dims), V[s,h] = W_UV[h] c_s (128 dims), rounded
 * to bf16; no other cache row is read.  Row r, head h then attends over the set of its valid idx
 * entries (idx [R, k] int32), or, with idx = NULL, over every position below row_len[r]
 * (dense causal: what the top-k selects when the row has at most k positions):
 *   z_s = softmax_scale * q[r,h,:] . K[row(s),h,:];  out[r,h,:] = softmax(z) . V;
 *   lse[r,h] = ln sum_s exp(z_s) (-inf for an empty set; lse may be NULL).
 * q: [R, n_heads, 192] bf16 (nope 128 | rope 64); kv: the latent cache, bf16 (contiguous
 * [N, 576] or paged [P, 64, 576]); w_uk, w_uv: [n_heads, 128, 512] bf16 (row d of head h is
 * the 512-vector producing key / value dim d); out: [R, n_heads, 128] bf16.  ws: device
 * scratch of dsa_mha_prefill_workspace_size(num_seqs, n_heads, R, max_row_len, idx != NULL)
 * bytes (the decompressed keys and values, 2 x 256 B per head for max_row_len positions of
 * each sequence, and the top-k masks), independent of the cache's size; needs no
 * initialisation; calls sharing a workspace must not run concurrently.
 * max_row_len <= 16384.  dsa_prefill_dense_mode(max_row_len, topk) is 1 when every row has
 * at most topk positions, i.e. when the dense mode (idx = NULL) equals DSA exactly.
 * Errors: DSA_ERR_INVALID_ARG for a bad row description, missing pointers, n_heads < 1,
 * a non-finite or non-positive scale, k outside [1, 2048] with idx; DSA_ERR_UNSUPPORTED for
 * max_row_len > 16384; DSA_ERR_WORKSPACE for a missing or small ws; DSA_ERR_HIP when a
 * launch fails. */
int dsa_prefill_dense_mode(int max_row_len, int topk);
size_t dsa_mha_prefill_workspace_size(int num_seqs, int n_heads, int num_rows, int max_row_len,
                                      int masked);
int dsa_mha_prefill(const dsa_rows *rows, int n_heads, float softmax_scale, const void *q,
                    const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx, int k,
                    void *out, float *lse, void *ws, size_t ws_bytes, void *stream);
int dsa_mha_prefill_paged(const dsa_rows *rows, int n_heads, float softmax_scale, const void *q,
                          const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx,
                          int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Prefill attention with the dispatch between its two forms ("DeepSeek-V3.2 技术报告摘要",
 * section 1: MLA in MQA mode over the top-k entries, and "短序列优化": short prefill as
 * masked MHA; the switch is the serving knob of "DeepSeek-V3.2" model docs, section 5.3,
 * SGLANG_NSA_PREFILL_DENSE_ATTN_KV_LEN_THRESHOLD, which the pages set to 0 there).
 * Inputs are those of dsa_indexer_topk(_paged) (idx_dtype .. topk, idx) and of
 * dsa_mha_prefill(_paged) (n_heads, softmax_scale, q [R, H, 192], kv, w_uk, w_uv, out
 * [R, H, 128], lse).  With max_row_len <= dense_threshold (and <= 16384) it runs the masked
 * MHA mode: dense causal when max_row_len <= topk (DSA selects every position; the indexer
 * does not run and logits / idx are not written), else over the top-k sets the indexer and
 * top-k write to logits / idx.  Otherwise (dense_threshold 0: always) it runs the MQA path:
 * indexer and top-k into logits / idx, the query absorbed through W_UK, q_abs[r,h] =
 * [W_UK[h]^T q_nope (512) | q_rope (64)] (bf16), dsa_sparse_mla_prefill(_paged) over idx with
 * d_qk 576 and d_v 512 (the latent, bf16), and out[r,h] = W_UV[h] o[r,h] (bf16); lse is the
 * attention's.  The two forms agree up to their bf16 roundings.
 * ws / ws_bytes: device scratch of dsa_sparse_attention_prefill_workspace_size(R, num_seqs,
 * max_row_len, idx_dtype, topk, n_heads, dense_threshold) bytes; needs no initialisation.
 * Errors: those of the calls it makes; DSA_ERR_UNSUPPORTED for the MQA path with
 * n_heads != 128. */
size_t dsa_sparse_attention_prefill_workspace_size(int num_rows, int num_seqs, int max_row_len,
                                                   int idx_dtype, int topk, int n_heads,
                                                   int dense_threshold);
int dsa_sparse_attention_prefill(const dsa_rows *rows, int idx_dtype, int idx_heads, int idx_dim,
                                 const void *q_idx, const float *q_idx_scale, const void *k_idx,
                                 const float *k_idx_scale, const float *w, float *logits,
                                 int64_t ld_logits, int topk, int32_t *idx, int n_heads,
                                 float softmax_scale, const void *q, const void *kv,
                                 const void *w_uk, const void *w_uv, void *out, float *lse,
                                 int dense_threshold, void *ws, size_t ws_bytes, void *stream);
int dsa_sparse_attention_prefill_paged(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                       int idx_dim, const void *q_idx, const float *q_idx_scale,
                                       const void *k_idx, const float *k_idx_scale,
                                       const float *w, float *logits, int64_t ld_logits, int topk,
                                       int32_t *idx, int n_heads, float softmax_scale,
                                       const void *q, const void *kv, const void *w_uk,
                                       const void *w_uv, void *out, float *lse,
                                       int dense_threshold, void *ws, size_t ws_bytes,
                                       void *stream);

/* ---------------------------------------------------------------------------------
 * Indexer-input and cache-write prep: the step in front of the indexer for every new token
 * ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ①: indexer keys and queries, FP8 supported;
 * "DeepSeek-V3.2-Exp" README, section "更新": the indexer's RoPE takes the non-interleaved
 * layout, the MLA's RoPE the interleaved one; "DeepSeek-V3.2" model docs, section 5.3: the
 * bf16 latent cache in 64-token pages).
 *
 * cos_sin: [max_position, 64] f32, row p = cos(p*theta_i) for i < 32, then sin(p*theta_i)
 *   for i < 32 (the caller's frequency schedule).
 * RoPE of a 64-dim part x at position p, pair i rotated by angle i of row p:
 *   indexer vectors (128 dims): dims 0..63, pairs (x[i], x[i+32])       (non-interleaved)
 *   MLA vectors (576 dims):     dims 512..575, pairs (x[512+2i], x[513+2i]) (interleaved)
 *   (a, b) -> (a cos - b sin, b cos + a sin), each product and sum one fp32 operation.
 * fp8 (idx_dtype DSA_FP8_E4M3): an indexer vector y is stored as e4m3 codes of y / scale
 *   (round to nearest even) with scale = max|y| / 448 (1 for a zero vector), as f32.
 * bf16 outputs are the rotated values rounded to nearest even; unrotated dims are copied.
 *
 * dsa_prep_cache_write: for each of num_tokens new tokens t at positions[t], writes cache
 *   row cache_rows[t] (the physical row: seq_start + position, or page * 64 + position % 64):
 *   k_idx_in [T, 128] bf16 -> k_idx_cache [num_cache_rows, 128] (bf16, or e4m3 with
 *   k_idx_scale [num_cache_rows] f32); kv_in [T, 576] bf16 -> kv_cache [num_cache_rows, 576]
 *   bf16.  Tokens with a position outside [0, max_position) or a row outside
 *   [0, num_cache_rows) are skipped (padding).  Two tokens naming one row race.
 * dsa_prep_queries: for each of num_rows query rows at positions[r]: q_idx_in [R, 64, 128]
 *   bf16 -> q_idx [R, 64, 128] (bf16, or e4m3 with q_idx_scale [R, 64] f32; q_idx may be
 *   q_idx_in for bf16), and the n_heads MLA heads of q [R, n_heads, 576] bf16 rotated in
 *   place.  Rows with a position outside [0, max_position) are left as they are.
 * All pointers are device pointers owned by the caller; the calls are asynchronous on
 * `stream`.  Errors: DSA_ERR_INVALID_ARG for negative counts, missing pointers, a scale
 * buffer missing for fp8 or given for bf16, max_position < 1, num_cache_rows < 1 or
 * n_heads < 1;
 * DSA_ERR_UNSUPPORTED for idx_dtype other than bf16 / fp8; num_tokens / num_rows == 0 is a
 * no-op. */
int dsa_prep_cache_write(int num_tokens, const int32_t *positions, const int64_t *cache_rows,
                         int64_t num_cache_rows, const float *cos_sin, int max_position,
                         int idx_dtype, const void *k_idx_in, void *k_idx_cache,
                         float *k_idx_scale, const void *kv_in, void *kv_cache, void *stream);
int dsa_prep_queries(int num_rows, const int32_t *positions, const float *cos_sin,
                     int max_position, int idx_dtype, const void *q_idx_in, void *q_idx,
                     float *q_idx_scale, int n_heads, void *q, void *stream);
/* Both of the above in one launch for num_tokens new tokens that are also the query rows
 * (decode, or a prefill chunk): positions[t] serves the key side and query row t. */
int dsa_prep(int num_tokens, const int32_t *positions, const int64_t *cache_rows,
             int64_t num_cache_rows, const float *cos_sin, int max_position, int idx_dtype,
             const void *k_idx_in, void *k_idx_cache, float *k_idx_scale, const void *kv_in,
             void *kv_cache, const void *q_idx_in, void *q_idx, float *q_idx_scale, int n_heads,
             void *q, void *stream);

/* ---------------------------------------------------------------------------------
 * Measurement aid (not a step of the method): the bf16 matrix-core rate the GPU sustains.
 * 512 workgroups of 4 waves (two per SIMD on every CU) each run `iters` rounds of 8
 * independent v_mfma_f32_16x16x32_bf16 on register operands; each wave writes one sum to
 * out[wave] so the work is kept.  Useful work: 2048 waves x iters x 8 x 16,384 flops; time
 * it with events on `stream` for the achievable bf16 MFMA rate at the clock the chip holds
 * under that load, to set beside the published peak.
 * out: device, DSA_MFMA_PROBE_WAVES floats.  iters: 1 .. 1,000,000, else DSA_ERR_INVALID_ARG. */
#define DSA_MFMA_PROBE_WAVES 2048
int dsa_mfma_rate_probe(int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
