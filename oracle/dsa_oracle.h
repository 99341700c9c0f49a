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

#ifdef __cplusplus
}
#endif
#endif
