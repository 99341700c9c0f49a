/*
 * dsa_oracle.h -- fp64 reference implementation of the DeepSeek Sparse
 * Attention (DSA) path: lightning indexer, top-k token selection and MLA in
 * MQA mode over the selected entries.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists to check the GPU library.  Only
 * the test-suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the GPU library.
 *
 * Sources (cited by page title and section):
 *  [R]  "DeepSeek-V3.2 技术报告摘要" (summary of the DeepSeek-V3.2 technical
 *       report), section 1 "预训练 Recipe", "关键设计：DeepSeek Sparse
 *       Attention (DSA)": ① Lightning Indexer (the I_{t,s} formula),
 *       ② Fine-grained Token Selection, and the paragraph on the MLA-based
 *       implementation (MQA mode, one latent entry shared by all heads).
 *  [M]  "DeepSeek-V3.2 -- Model techniques map", table "Checked in its code":
 *       rows "Indexer-selected sparse attention", "Multi-head latent
 *       attention", "Partial RoPE", "Learnable attention sink", "Gated
 *       attention output".
 *  [S]  "DeepSeek-V3.2" (miles model docs), section 1 "Model Introduction"
 *       (shapes) and section 5.3 "Rollout & SGLang" (bf16 cache, page 64).
 *  [E]  "DeepSeek-V3.2-Exp" README, section "更新" (the 2025-11-17 update):
 *       the indexer's RoPE takes its input in the non-interleaved layout, the
 *       MLA's RoPE in the interleaved layout.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element encodings of the inputs */
enum { OREF_F32 = 0, OREF_BF16 = 1, OREF_E4M3 = 2 };

/* Where query row r looks: sequence row_seq[r], positions [0, row_len[r]).
 * Exactly one of seq_start (contiguous cache) / page_table (paged cache). */
typedef struct {
    int32_t        n_rows;
    const int32_t *row_seq;     /* [n_rows] */
    const int32_t *row_len;     /* [n_rows] */
    const int64_t *seq_start;   /* [n_seqs] first cache row of a sequence, or NULL */
    const int32_t *page_table;  /* [n_seqs * max_pages], or NULL */
    int32_t        max_pages;
    int32_t        page_size;
} oref_rows;

void oref_bf16_to_f64(const uint16_t *src, double *dst, int64_t n);
void oref_e4m3_to_f64(const uint8_t *src, double *dst, int64_t n);

/* Cache row holding position s of sequence b. */
int64_t oref_cache_row(const oref_rows *rows, int32_t b, int64_t s);

/* Indexer scores for the query rows listed in which[0..n_which).
 * out row i (stride ld) holds I[which[i], s] for s < row_len; the rest untouched. */
int oref_indexer(int dtype, int n_heads, int head_dim,
                 const void *q, const float *q_scale, const float *w,
                 const void *k, const float *k_scale,
                 const oref_rows *rows, const int32_t *which, int32_t n_which,
                 double *out, int64_t ld, int n_threads);

/* Top-k of one score row: writes the k_eff = min(k, n) selected positions in
 * ascending order, then -1 up to k.  Returns k_eff. */
int oref_topk_row(const double *x, int64_t n, int32_t k, int32_t *out);
int oref_topk_rows(const double *x, int64_t ld, const int32_t *len, int32_t n_rows,
                   int32_t k, int32_t *out, int n_threads);
int oref_topk_rows_f32(const float *x, int64_t ld, const int32_t *len, int32_t n_rows,
                       int32_t k, int32_t *out, int n_threads);

/* Sparse MLA in MQA mode over the idx entries of each listed row; out is
 * [n_which, H, Dv], lse [n_which, H] (natural log; -inf for an empty set). */
int oref_sparse_mla(int dtype, int n_heads, int d_qk, int d_v, double scale,
                    const void *q, const void *kv, const int32_t *idx, int32_t k,
                    const oref_rows *rows, const int32_t *which, int32_t n_which,
                    double *out, double *lse, int n_threads);

/* Dense causal MQA: the same attention over every position [0, row_len). */
int oref_dense_mqa(int dtype, int n_heads, int d_qk, int d_v, double scale,
                   const void *q, const void *kv,
                   const oref_rows *rows, const int32_t *which, int32_t n_which,
                   double *out, double *lse, int n_threads);

/* ------------------------------------------------------------------------ */
/* Indexer-input and cache-write prep ([E] RoPE layouts, [R] ① FP8 indexer,  */
/* [S] 5.3 cache).  These steps end in a rounding decision (a bf16 or e4m3   */
/* code), so they are computed in fp32 exactly as defined below, each       */
/* operation rounded once (no fused multiply-add), and the codes chosen      */
/* from the definitions of the formats.                                      */
/*                                                                           */
/* cos_sin row p (p < max_pos) holds cos(p*theta_i) for i < 32, then         */
/* sin(p*theta_i) for i < 32: the caller's frequency schedule.               */
/* RoPE on a 64-dim part x, pair i (i < 32) rotated by angle i of the row:    */
/*   non-interleaved: (x[i], x[i+32])     interleaved: (x[2i], x[2i+1])      */
/*   (a, b) -> (a*cos - b*sin, b*cos + a*sin)                                */
/* Indexer vectors (128 dims): dims 0..63 carry the rotation, 64..127 not.   */
/* MLA vectors (576 dims): dims 512..575 carry the rotation.                 */
/* fp8 quantisation of a 128-dim vector y: amax = max |y_j|,                  */
/*   scale = amax / 448 (1 when amax = 0), code_j = e4m3 nearest to          */
/*   y_j / scale, ties to the even code.                                     */
/* ------------------------------------------------------------------------ */

/* fp32 -> bf16 code: the nearest bf16 value, ties to the even code. */
uint16_t oref_bf16_code(float f);
/* fp32 -> OCP E4M3FN code: the nearest finite e4m3 value (|v| <= 448),
 * ties to the even code; values beyond 448 take 448. */
uint8_t oref_e4m3_code(float f);
void oref_bf16_codes(const float *src, uint16_t *dst, int64_t n);
void oref_e4m3_codes(const float *src, uint8_t *dst, int64_t n);

/* Key side, per new token t: the indexer key k_in[t] (bf16, 128 dims) rotated
 * (non-interleaved) and written to k_cache row rows_out[t] as bf16
 * (idx_dtype OREF_BF16) or as e4m3 codes plus k_scale[row] (OREF_E4M3); the
 * MLA entry kv_in[t] (bf16, 576 dims) with its last 64 dims rotated
 * (interleaved) written to kv_cache row rows_out[t].  Tokens whose position is
 * outside [0, max_pos) or whose row is outside [0, cache_rows) are skipped. */
int oref_prep_keys(int32_t n_tok, const int32_t *pos, const int64_t *rows_out, int64_t cache_rows,
                   const float *cos_sin, int32_t max_pos, int idx_dtype,
                   const uint16_t *k_in, void *k_cache, float *k_scale,
                   const uint16_t *kv_in, uint16_t *kv_cache);

/* Query side, per row r at position pos[r]: each of the n_idx_heads indexer
 * heads of qi_in[r] (bf16, 128 dims) rotated (non-interleaved) and written as
 * bf16, or as e4m3 codes with qi_scale[r, head]; each of the n_heads MLA heads
 * of q[r] (bf16, 576 dims) rotated in place on its last 64 dims
 * (interleaved).  Rows with a position outside [0, max_pos) are skipped. */
int oref_prep_queries(int32_t n_rows, const int32_t *pos, const float *cos_sin, int32_t max_pos,
                      int idx_dtype, int32_t n_idx_heads, const uint16_t *qi_in, void *qi_out,
                      float *qi_scale, int32_t n_heads, uint16_t *q);

/* ------------------------------------------------------------------------ */
/* Masked MHA mode for short prefill ([R] "短序列优化"; [M] "Multi-head      */
/* latent attention").  Decompression, per cache row n and head h:           */
/*   k[n,h] = [W_UK[h] . c_n (128) | kr_n (64)],  v[n,h] = W_UV[h] . c_n (128) */
/* with kv rows [c_n (512) | kr_n (64)] bf16 and W_UK, W_UV [H, 128, 512]     */
/* bf16; k, v in fp64 [rows, H, 192] / [rows, H, 128].                       */
/* Attention of row r, head h over the set of its valid idx entries (idx     */
/* [R, topk]), or over every position below row_len when idx is NULL:        */
/*   z_s = scale * q[r,h] . k[row(s),h];  out = softmax(z) . v;  lse = ln sum */
/* q is [R, H, 192] bf16; out [n_which, H, 128], lse [n_which, H].          */
/* ------------------------------------------------------------------------ */
int oref_mha_decompress(int32_t n_cache_rows, int n_heads, const uint16_t *kv, const uint16_t *w_uk,
                        const uint16_t *w_uv, double *k, double *v, int n_threads);
int oref_mha(int n_heads, const uint16_t *q, const double *k, const double *v,
             const oref_rows *rows, const int32_t *idx, int32_t topk, double scale,
             const int32_t *which, int32_t n_which, double *out, double *lse, int n_threads);

#ifdef __cplusplus
}
#endif
#endif
