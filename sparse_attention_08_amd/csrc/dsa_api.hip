// dsa_api.hip -- the C ABI declared in include/dsa.h: argument validation (all of it on
// the host, before anything is enqueued) and dispatch to the kernel launchers.
#include "dsa.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "dsa_launch.h"

namespace {

using dsa::RowsHost;

bool rows_ok(const dsa_rows *rows, bool paged) {
  if (!rows) return false;
  if (rows->num_rows < 0 || rows->num_seqs < 1) return false;
  if (rows->num_rows == 0) return true;
  if (!rows->row_seq || !rows->row_len || rows->max_row_len < 1) return false;
  if (paged) {
    if (!rows->page_table || rows->seq_start) return false;
    if (rows->page_size != DSA_PAGE_SIZE) return false;
    if (rows->max_pages < (rows->max_row_len + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE) return false;
  } else {
    if (!rows->seq_start || rows->page_table) return false;
  }
  return true;
}

RowsHost to_host(const dsa_rows *rows) {
  return RowsHost{rows->num_rows,  rows->num_seqs,  rows->row_seq,   rows->row_len,
                  rows->max_row_len, rows->seq_start, rows->page_table, rows->max_pages};
}

int status_of(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Host-side checks of an indexer call; DSA_OK means the call may proceed (or is empty).
int indexer_check(const dsa_rows *rows, bool paged, int dtype, int n_heads, int head_dim,
                  const void *q, const float *q_scale, const void *k, const float *k_scale,
                  const float *w, float *logits, int64_t ld_logits) {
  if (!rows_ok(rows, paged)) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (n_heads <= 0 || head_dim <= 0) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !k || !w || !logits) return DSA_ERR_INVALID_ARG;
  if (ld_logits < rows->max_row_len) return DSA_ERR_INVALID_ARG;
  const bool fp8 = dtype == DSA_FP8_E4M3;
  if (fp8 != (q_scale != nullptr) || fp8 != (k_scale != nullptr)) return DSA_ERR_INVALID_ARG;
  if (dtype == DSA_F32) {
    if (n_heads > 64 || head_dim > 256) return DSA_ERR_UNSUPPORTED;
  } else if (n_heads != 64 || head_dim != 128) {
    return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

// bf16 batches with many rows per sequence (prefill, chunked prefill, multi-token decode)
// take the indexer whose workgroups share key tiles between 8 consecutive rows: from 8 rows
// per sequence on average, or from 4 over contexts of at most 32K.  Measured on MI355X
// against the one-row-at-a-time indexer (whose key loads stay in cache when rows share
// sequences): 8K contexts x 4 rows 39 vs 52 us, 128K x 4 rows 58 vs 51 us, 32K x 16 rows 80
// vs 96 us, 128K x 2 rows 87 vs 53 us.  fp8 batches always take the one-row-at-a-time
// indexer, which measured faster at every shape tried.
bool shares_keys(const dsa_rows *rows, int dtype) {
  if (dtype != DSA_BF16) return false;
  const int64_t r = rows->num_rows, s = rows->num_seqs;
  return r >= 8 * s || (r >= 4 * s && rows->max_row_len <= 32768);
}

hipError_t indexer_launch(const dsa_rows *rows, bool paged, int dtype, int n_heads, int head_dim,
                          const void *q, const float *q_scale, const void *k, const float *k_scale,
                          const float *w, float *logits, int64_t ld_logits, hipStream_t s) {
  const RowsHost rh = to_host(rows);
  if (dtype == DSA_F32)
    return dsa::launch_indexer_f32(rh, paged, n_heads, head_dim, static_cast<const float *>(q),
                                   static_cast<const float *>(k), w, logits, ld_logits, s);
  if (shares_keys(rows, dtype))
    return dsa::launch_indexer_prefill(rh, paged, q, k, w, logits, ld_logits, s);
  return dsa::launch_indexer_mfma(rh, paged, dtype == DSA_FP8_E4M3, q, q_scale, k, k_scale, w,
                                  logits, ld_logits, s);
}

int indexer_common(const dsa_rows *rows, bool paged, int dtype, int n_heads, int head_dim,
                   const void *q, const float *q_scale, const void *k, const float *k_scale,
                   const float *w, float *logits, int64_t ld_logits, void *stream) {
  const int st = indexer_check(rows, paged, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                               logits, ld_logits);
  if (st != DSA_OK || rows->num_rows == 0) return st;
  return status_of(indexer_launch(rows, paged, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                                  logits, ld_logits, static_cast<hipStream_t>(stream)));
}

// Histogram lists per row when the per-row indexer's workgroups feed the top-k directly, or 0
// when the batch takes the separate path (f32 indexer, the one-workgroup-per-row top-k
// schedule, or the shared-key indexer).
int hist_lists_of_shape(int num_rows, int max_row_len, int dtype) {
  if (dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return 0;
  const int nh = dsa::indexer_blocks_per_row(num_rows, max_row_len, dtype == DSA_FP8_E4M3);
  return dsa::topk_hist_fusable(num_rows, max_row_len, nh) ? nh : 0;
}
int fused_hist_lists(const dsa_rows *rows, int dtype) {
  if (shares_keys(rows, dtype)) return 0;
  return hist_lists_of_shape(rows->num_rows, rows->max_row_len, dtype);
}

// Workspace of the indexer + top-k for any batch of this shape: the size queries do not see
// the number of sequences, so this covers both the fused and the separate top-k.
size_t indexer_topk_ws(int num_rows, int max_row_len, int dtype, int k) {
  const size_t sep = dsa::topk_workspace_bytes(num_rows, max_row_len, k);
  const int nh = hist_lists_of_shape(num_rows, max_row_len, dtype);
  return nh ? std::max(sep, dsa::topk_fused_workspace_bytes(num_rows, max_row_len, nh)) : sep;
}

int indexer_topk_common(const dsa_rows *rows, bool paged, int dtype, int n_heads, int head_dim,
                        const void *q, const float *q_scale, const void *k, const float *k_scale,
                        const float *w, float *logits, int64_t ld_logits, int topk, int32_t *idx,
                        void *ws, size_t ws_bytes, void *stream) {
  const int st = indexer_check(rows, paged, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                               logits, ld_logits);
  if (st != DSA_OK) return st;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!idx) return DSA_ERR_INVALID_ARG;
  const size_t need = indexer_topk_ws(rows->num_rows, rows->max_row_len, dtype, topk);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = rows->num_rows, L = rows->max_row_len;
  const int nh = fused_hist_lists(rows, dtype);
  if (nh) {
    const dsa::TopkHistDest dest = dsa::topk_hist_dest(ws, R, L, nh);
    hipError_t e = dsa::launch_indexer_mfma_hist(to_host(rows), paged, dtype == DSA_FP8_E4M3, q,
                                                 q_scale, k, k_scale, w, logits, ld_logits, dest, s);
    if (e != hipSuccess) return DSA_ERR_HIP;
    return status_of(dsa::launch_topk_after_hist(logits, ld_logits, rows->row_len, R, L, topk, idx,
                                                 ws, nh, s));
  }
  hipError_t e = indexer_launch(rows, paged, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                                logits, ld_logits, s);
  if (e != hipSuccess) return DSA_ERR_HIP;
  return status_of(dsa::launch_topk(logits, ld_logits, rows->row_len, R, L, topk, idx, ws, s));
}

enum class MlaMode { kDecode, kPrefill };

int mla_common(const dsa_rows *rows, bool paged, MlaMode mode, int dtype, int n_heads, int d_qk,
               int d_v, float softmax_scale, const void *q, const void *kv, const int32_t *idx,
               int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!rows_ok(rows, paged)) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (n_heads <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk) return DSA_ERR_INVALID_ARG;
  if (k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !kv || !idx || !out) return DSA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RowsHost rh = to_host(rows);
  if (dtype == DSA_F32) {
    if (n_heads > 128 || d_qk > 256 || d_v > 256) return DSA_ERR_UNSUPPORTED;
    return status_of(dsa::launch_mla_f32(rh, paged, n_heads, d_qk, d_v, softmax_scale,
                                         static_cast<const float *>(q),
                                         static_cast<const float *>(kv), idx, k,
                                         static_cast<float *>(out), lse, s));
  }
  if (dtype != DSA_BF16) return DSA_ERR_UNSUPPORTED;
  if (n_heads != 128 || d_qk != 576 || d_v != 512) return DSA_ERR_UNSUPPORTED;
  int splits = 1;
  if (mode == MlaMode::kDecode) {
    splits = dsa::mla_num_splits(rows->num_rows, n_heads, k);
    const size_t need = dsa::mla_workspace_bytes(rows->num_rows, n_heads, d_v, k);
    if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  }
  return status_of(dsa::launch_mla_bf16(rh, paged, n_heads, softmax_scale, q, kv, idx, k, out, lse,
                                        splits, ws, s));
}

// Stages 1-3 of a decode batch.  Up to kSelectInAttentionRows long rows (batches whose
// indexer feeds the top-k histograms) with the bf16 attention finish the selection inside
// the attention workgroups; every other batch runs the two calls in turn.  Each split of a
// row repeats the row's selection, which pays while the saved launch outweighs the longer
// attention prologue (measured: 8 rows of 128K gain, 32 rows of up to 64K lose).
constexpr int kSelectInAttentionRows = 16;
bool decode_fusable(const dsa_rows *rows, int idx_dtype, int dtype) {
  return dtype == DSA_BF16 && rows->num_rows <= kSelectInAttentionRows &&
         fused_hist_lists(rows, idx_dtype) > 0;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_ws(int num_rows, int max_row_len, int idx_dtype, int topk, int n_heads, int d_v) {
  return align256(indexer_topk_ws(num_rows, max_row_len, idx_dtype, topk)) +
         dsa::mla_workspace_bytes(num_rows, n_heads, d_v, topk);
}

int attention_decode_common(const dsa_rows *rows, bool paged, int idx_dtype, int idx_heads,
                            int idx_dim, const void *q_idx, const float *q_idx_scale,
                            const void *k_idx, const float *k_idx_scale, const float *w,
                            float *logits, int64_t ld_logits, int topk, int32_t *idx, int dtype,
                            int n_heads, int d_qk, int d_v, float softmax_scale, const void *q,
                            const void *kv, void *out, float *lse, void *ws, size_t ws_bytes,
                            void *stream) {
  int st = indexer_check(rows, paged, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale, k_idx,
                         k_idx_scale, w, logits, ld_logits);
  if (st != DSA_OK) return st;
  if (topk < 1 || topk > DSA_MAX_TOPK) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (n_heads <= 0 || d_qk <= 0 || d_v <= 0 || d_v > d_qk) return DSA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!idx || !q || !kv || !out) return DSA_ERR_INVALID_ARG;
  if (dtype == DSA_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
  if (dtype == DSA_F32 && (n_heads > 128 || d_qk > 256 || d_v > 256)) return DSA_ERR_UNSUPPORTED;
  if (dtype == DSA_BF16 && (n_heads != 128 || d_qk != 576 || d_v != 512))
    return DSA_ERR_UNSUPPORTED;
  const int R = rows->num_rows, L = rows->max_row_len;
  const size_t tk_bytes = align256(indexer_topk_ws(R, L, idx_dtype, topk));
  const size_t need = decode_ws(R, L, idx_dtype, topk, n_heads, d_v);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  void *tk_ws = tk_bytes ? wsb : nullptr;
  void *ml_ws = need > tk_bytes ? wsb + tk_bytes : nullptr;
  const size_t ml_bytes = need - tk_bytes;
  if (!decode_fusable(rows, idx_dtype, dtype)) {
    st = indexer_topk_common(rows, paged, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale, k_idx,
                             k_idx_scale, w, logits, ld_logits, topk, idx, tk_ws, tk_bytes, stream);
    if (st != DSA_OK) return st;
    return mla_common(rows, paged, MlaMode::kDecode, dtype, n_heads, d_qk, d_v, softmax_scale, q,
                      kv, idx, topk, out, lse, ml_ws, ml_bytes, stream);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nh = fused_hist_lists(rows, idx_dtype);
  const dsa::TopkHistDest dest = dsa::topk_hist_dest(tk_ws, R, L, nh);
  hipError_t e = dsa::launch_indexer_mfma_hist(to_host(rows), paged, idx_dtype == DSA_FP8_E4M3,
                                               q_idx, q_idx_scale, k_idx, k_idx_scale, w, logits,
                                               ld_logits, dest, s);
  if (e == hipSuccess)
    e = dsa::launch_topk_filter_after_hist(logits, ld_logits, rows->row_len, R, L, topk, idx,
                                           tk_ws, nh, s);
  if (e == hipSuccess)
    e = dsa::launch_mla_bf16_select(to_host(rows), paged, n_heads, softmax_scale, q, kv, idx, topk,
                                    out, lse, dsa::mla_num_splits(R, n_heads, topk), ml_ws,
                                    logits, ld_logits, tk_ws, nh, s);
  return status_of(e);
}

constexpr int kMhaMaxRowLen = 16384;   // the attended range's pages are staged in LDS

int mha_common(const dsa_rows *rows, bool paged, int n_heads, float softmax_scale, const void *q,
               const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx, int k,
               void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  if (!rows_ok(rows, paged)) return DSA_ERR_INVALID_ARG;
  if (n_heads < 1) return DSA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (idx && (k < 1 || k > DSA_MAX_TOPK)) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !kv || !w_uk || !w_uv || !out) return DSA_ERR_INVALID_ARG;
  if (rows->max_row_len > kMhaMaxRowLen) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa::mha_workspace_bytes(rows->num_seqs, n_heads, rows->num_rows,
                                               rows->max_row_len, idx != nullptr);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  return status_of(dsa::launch_mha_prefill(to_host(rows), paged, n_heads, softmax_scale, q, kv,
                                           w_uk, w_uv, idx, k, out, lse, ws,
                                           static_cast<hipStream_t>(stream)));
}

// The prefill dispatch: the masked MHA mode when the batch's longest row reaches at most
// dense_threshold positions (and the mode's 16384 limit), else the MQA path.  The MHA mode
// needs the selection only for rows longer than topk.
bool prefill_uses_mha(int max_row_len, int dense_threshold) {
  return max_row_len <= dense_threshold && max_row_len <= kMhaMaxRowLen;
}

size_t prefill_ws(int R, int B, int L, int idx_dtype, int topk, int H, int dense_threshold) {
  const bool mha = prefill_uses_mha(L, dense_threshold);
  const size_t sel = (mha && L <= topk) ? 0 : align256(indexer_topk_ws(R, L, idx_dtype, topk));
  return sel + (mha ? dsa::mha_workspace_bytes(B, H, R, L, L > topk)
                    : dsa::absorb_workspace_bytes(R, H));
}

int prefill_common(const dsa_rows *rows, bool paged, int idx_dtype, int idx_heads, int idx_dim,
                   const void *q_idx, const float *q_idx_scale, const void *k_idx,
                   const float *k_idx_scale, const float *w, float *logits, int64_t ld_logits,
                   int topk, int32_t *idx, int n_heads, float softmax_scale, const void *q,
                   const void *kv, const void *w_uk, const void *w_uv, void *out, float *lse,
                   int dense_threshold, void *ws, size_t ws_bytes, void *stream) {
  if (!rows_ok(rows, paged)) return DSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > DSA_MAX_TOPK || n_heads < 1) return DSA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !kv || !w_uk || !w_uv || !out) return DSA_ERR_INVALID_ARG;
  const int R = rows->num_rows, L = rows->max_row_len;
  const bool mha = prefill_uses_mha(L, dense_threshold);
  const bool select = !mha || L > topk;
  if (select) {
    const int st = indexer_check(rows, paged, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale,
                                 k_idx, k_idx_scale, w, logits, ld_logits);
    if (st != DSA_OK) return st;
    if (!idx) return DSA_ERR_INVALID_ARG;
  }
  if (!mha && n_heads != 128) return DSA_ERR_UNSUPPORTED;   // the bf16 MQA attention's heads
  const size_t need = prefill_ws(R, rows->num_seqs, L, idx_dtype, topk, n_heads, dense_threshold);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  const size_t sel_bytes = select ? align256(indexer_topk_ws(R, L, idx_dtype, topk)) : 0;
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  if (select) {
    const int st = indexer_topk_common(rows, paged, idx_dtype, idx_heads, idx_dim, q_idx,
                                       q_idx_scale, k_idx, k_idx_scale, w, logits, ld_logits,
                                       topk, idx, sel_bytes ? wsb : nullptr, sel_bytes, stream);
    if (st != DSA_OK) return st;
  }
  if (mha)
    return mha_common(rows, paged, n_heads, softmax_scale, q, kv, w_uk, w_uv,
                      select ? idx : nullptr, topk, out, lse, wsb + sel_bytes, need - sel_bytes,
                      stream);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dsa::AbsorbBuffers ab = dsa::carve_absorb(wsb + sel_bytes, R, n_heads);
  hipError_t e = dsa::launch_absorb_query(R, n_heads, q, w_uk, ab, s);
  if (e != hipSuccess) return DSA_ERR_HIP;
  const int st = mla_common(rows, paged, MlaMode::kPrefill, DSA_BF16, n_heads, 576, 512,
                            softmax_scale, ab.q_abs, kv, idx, topk, ab.o_lat, lse, nullptr, 0,
                            stream);
  if (st != DSA_OK) return st;
  return status_of(dsa::launch_expand_output(R, n_heads, ab.o_lat, w_uv, out, s));
}

int prep_keys_check(const dsa::PrepKeys &k, bool fp8) {
  if (k.T < 0 || k.cache_rows < 1) return DSA_ERR_INVALID_ARG;
  if (k.T == 0) return DSA_OK;
  if (!k.pos || !k.rows || !k.k_in || !k.k_cache || !k.kv_in || !k.kv_cache)
    return DSA_ERR_INVALID_ARG;
  return (fp8 != (k.k_scale != nullptr)) ? DSA_ERR_INVALID_ARG : DSA_OK;
}

int prep_queries_check(const dsa::PrepQueries &q, bool fp8) {
  if (q.R < 0 || q.n_heads < 1) return DSA_ERR_INVALID_ARG;
  if (q.R == 0) return DSA_OK;
  if (!q.pos || !q.qi_in || !q.qi_out || !q.q) return DSA_ERR_INVALID_ARG;
  return (fp8 != (q.qi_scale != nullptr)) ? DSA_ERR_INVALID_ARG : DSA_OK;
}

int prep_common(const dsa::PrepKeys &keys, const dsa::PrepQueries &queries, const float *cos_sin,
                int max_position, int idx_dtype, void *stream) {
  if (max_position < 1) return DSA_ERR_INVALID_ARG;
  if (idx_dtype != DSA_F32 && idx_dtype != DSA_BF16 && idx_dtype != DSA_FP8_E4M3)
    return DSA_ERR_INVALID_ARG;
  const bool fp8 = idx_dtype == DSA_FP8_E4M3;
  int st = prep_keys_check(keys, fp8);
  if (st == DSA_OK) st = prep_queries_check(queries, fp8);
  if (st != DSA_OK) return st;
  if (idx_dtype == DSA_F32) return DSA_ERR_UNSUPPORTED;
  if (keys.T == 0 && queries.R == 0) return DSA_OK;
  if (!cos_sin) return DSA_ERR_INVALID_ARG;
  return status_of(dsa::launch_prep(queries, keys, cos_sin, max_position, fp8,
                                    static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char *dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape/dtype combination not supported";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP launch failed";
    default: return "unknown dsa status";
  }
}

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

int dsa_indexer_logits(const dsa_rows *rows, int dtype, int n_heads, int head_dim, const void *q,
                       const float *q_scale, const void *k, const float *k_scale, const float *w,
                       float *logits, int64_t ld_logits, void *stream) {
  return indexer_common(rows, false, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w, logits,
                        ld_logits, stream);
}

int dsa_indexer_logits_paged(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                             const void *q, const float *q_scale, const void *k,
                             const float *k_scale, const float *w, float *logits,
                             int64_t ld_logits, void *stream) {
  return indexer_common(rows, true, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w, logits,
                        ld_logits, stream);
}

size_t dsa_indexer_topk_workspace_size(int num_rows, int max_row_len, int dtype, int k) {
  if (num_rows < 0 || max_row_len < 1 || k < 1 || k > DSA_MAX_TOPK) return 0;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return 0;
  return indexer_topk_ws(num_rows, max_row_len, dtype, k);
}

int dsa_indexer_topk(const dsa_rows *rows, int dtype, int n_heads, int head_dim, const void *q,
                     const float *q_scale, const void *k, const float *k_scale, const float *w,
                     float *logits, int64_t ld_logits, int topk, int32_t *idx, void *ws,
                     size_t ws_bytes, void *stream) {
  return indexer_topk_common(rows, false, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                             logits, ld_logits, topk, idx, ws, ws_bytes, stream);
}

int dsa_indexer_topk_paged(const dsa_rows *rows, int dtype, int n_heads, int head_dim,
                           const void *q, const float *q_scale, const void *k,
                           const float *k_scale, const float *w, float *logits, int64_t ld_logits,
                           int topk, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
  return indexer_topk_common(rows, true, dtype, n_heads, head_dim, q, q_scale, k, k_scale, w,
                             logits, ld_logits, topk, idx, ws, ws_bytes, stream);
}

size_t dsa_topk_workspace_size(int num_rows, int max_row_len, int k) {
  if (num_rows < 0 || max_row_len < 1 || k < 1 || k > DSA_MAX_TOPK) return 0;
  return dsa::topk_workspace_bytes(num_rows, max_row_len, k);
}

int dsa_topk(const float *logits, int64_t ld_logits, const int32_t *row_len, int num_rows,
             int max_row_len, int k, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
  if (num_rows < 0 || max_row_len < 1 || k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_INVALID_ARG;
  if (num_rows == 0) return DSA_OK;
  if (!logits || !row_len || !idx || ld_logits < max_row_len) return DSA_ERR_INVALID_ARG;
  const size_t need = dsa::topk_workspace_bytes(num_rows, max_row_len, k);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  return status_of(dsa::launch_topk(logits, ld_logits, row_len, num_rows, max_row_len, k, idx, ws,
                                    static_cast<hipStream_t>(stream)));
}

size_t dsa_sparse_mla_workspace_size(int num_rows, int n_heads, int d_v, int k) {
  if (num_rows < 1 || n_heads < 1 || d_v < 1 || k < 1 || k > DSA_MAX_TOPK) return 0;
  return dsa::mla_workspace_bytes(num_rows, n_heads, d_v, k);
}

int dsa_sparse_mla_decode(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                          float softmax_scale, const void *q, const void *kv, const int32_t *idx,
                          int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  return mla_common(rows, false, MlaMode::kDecode, dtype, n_heads, d_qk, d_v, softmax_scale, q, kv,
                    idx, k, out, lse, ws, ws_bytes, stream);
}

int dsa_sparse_mla_decode_paged(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                                float softmax_scale, const void *q, const void *kv,
                                const int32_t *idx, int k, void *out, float *lse, void *ws,
                                size_t ws_bytes, void *stream) {
  return mla_common(rows, true, MlaMode::kDecode, dtype, n_heads, d_qk, d_v, softmax_scale, q, kv,
                    idx, k, out, lse, ws, ws_bytes, stream);
}

size_t dsa_sparse_attention_decode_workspace_size(int num_rows, int max_row_len, int idx_dtype,
                                                  int topk, int n_heads, int d_v) {
  if (num_rows < 1 || max_row_len < 1 || topk < 1 || topk > DSA_MAX_TOPK || n_heads < 1 || d_v < 1)
    return 0;
  if (idx_dtype != DSA_F32 && idx_dtype != DSA_BF16 && idx_dtype != DSA_FP8_E4M3) return 0;
  return decode_ws(num_rows, max_row_len, idx_dtype, topk, n_heads, d_v);
}

int dsa_sparse_attention_decode(const dsa_rows *rows, int idx_dtype, int idx_heads, int idx_dim,
                                const void *q_idx, const float *q_idx_scale, const void *k_idx,
                                const float *k_idx_scale, const float *w, float *logits,
                                int64_t ld_logits, int topk, int32_t *idx, int dtype, int n_heads,
                                int d_qk, int d_v, float softmax_scale, const void *q,
                                const void *kv, void *out, float *lse, void *ws, size_t ws_bytes,
                                void *stream) {
  return attention_decode_common(rows, false, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale,
                                 k_idx, k_idx_scale, w, logits, ld_logits, topk, idx, dtype,
                                 n_heads, d_qk, d_v, softmax_scale, q, kv, out, lse, ws, ws_bytes,
                                 stream);
}

// ---- the decode call without a workspace argument --------------------------------
// Its scratch is this file-scope device array: every GPU the library runs on holds one copy
// from the library's load until the process ends.  Host code never uses the array's name as
// an address (on the host it only names the symbol): the device address is looked up once
// per device, with that device current, and kept.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];   // device address of `scratch` per device (null: not yet)

// The current device's copy of `scratch` (looked up on the first call on that device).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DSA_OK;
}

}  // namespace

int dsa_sparse_attention_decode_noalloc(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                        int idx_dim, const void *q_idx, const float *q_idx_scale,
                                        const void *k_idx, const float *k_idx_scale,
                                        const float *w, float *logits, int64_t ld_logits, int topk,
                                        int32_t *idx, int dtype, int n_heads, int d_qk, int d_v,
                                        float softmax_scale, const void *q, const void *kv,
                                        void *out, float *lse, void *stream) {
  if (!rows) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows > 0 &&
      dsa_sparse_attention_decode_workspace_size(rows->num_rows, rows->max_row_len, idx_dtype, topk,
                                                 n_heads, d_v) > DSA_NOALLOC_SCRATCH_BYTES)
    return DSA_ERR_WORKSPACE;   // the batch needs more scratch than the static array holds
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != DSA_OK) return st;
  return attention_decode_common(rows, false, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale,
                                 k_idx, k_idx_scale, w, logits, ld_logits, topk, idx, dtype,
                                 n_heads, d_qk, d_v, softmax_scale, q, kv, out, lse, ws,
                                 DSA_NOALLOC_SCRATCH_BYTES, stream);
}

int dsa_sparse_attention_decode_paged(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                      int idx_dim, const void *q_idx, const float *q_idx_scale,
                                      const void *k_idx, const float *k_idx_scale, const float *w,
                                      float *logits, int64_t ld_logits, int topk, int32_t *idx,
                                      int dtype, int n_heads, int d_qk, int d_v,
                                      float softmax_scale, const void *q, const void *kv,
                                      void *out, float *lse, void *ws, size_t ws_bytes,
                                      void *stream) {
  return attention_decode_common(rows, true, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale,
                                 k_idx, k_idx_scale, w, logits, ld_logits, topk, idx, dtype,
                                 n_heads, d_qk, d_v, softmax_scale, q, kv, out, lse, ws, ws_bytes,
                                 stream);
}

int dsa_sparse_mla_prefill(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                           float softmax_scale, const void *q, const void *kv, const int32_t *idx,
                           int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  return mla_common(rows, false, MlaMode::kPrefill, dtype, n_heads, d_qk, d_v, softmax_scale, q,
                    kv, idx, k, out, lse, nullptr, 0, stream);
}

int dsa_sparse_mla_prefill_paged(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                                 float softmax_scale, const void *q, const void *kv,
                                 const int32_t *idx, int k, void *out, float *lse, void *ws,
                                 size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  return mla_common(rows, true, MlaMode::kPrefill, dtype, n_heads, d_qk, d_v, softmax_scale, q,
                    kv, idx, k, out, lse, nullptr, 0, stream);
}

int dsa_prefill_dense_mode(int max_row_len, int topk) {
  return (max_row_len >= 1 && topk >= 1 && max_row_len <= topk) ? 1 : 0;
}

size_t dsa_mha_prefill_workspace_size(int num_seqs, int n_heads, int num_rows, int max_row_len,
                                      int masked) {
  if (num_seqs < 1 || n_heads < 1 || num_rows < 0 || max_row_len < 1) return 0;
  return dsa::mha_workspace_bytes(num_seqs, n_heads, num_rows, max_row_len, masked != 0);
}

int dsa_mha_prefill(const dsa_rows *rows, int n_heads, float softmax_scale, const void *q,
                    const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx, int k,
                    void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  return mha_common(rows, false, n_heads, softmax_scale, q, kv, w_uk, w_uv, idx, k, out, lse, ws,
                    ws_bytes, stream);
}

int dsa_mha_prefill_paged(const dsa_rows *rows, int n_heads, float softmax_scale, const void *q,
                          const void *kv, const void *w_uk, const void *w_uv, const int32_t *idx,
                          int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  return mha_common(rows, true, n_heads, softmax_scale, q, kv, w_uk, w_uv, idx, k, out, lse, ws,
                    ws_bytes, stream);
}

size_t dsa_sparse_attention_prefill_workspace_size(int num_rows, int num_seqs, int max_row_len,
                                                   int idx_dtype, int topk, int n_heads,
                                                   int dense_threshold) {
  if (num_rows < 0 || num_seqs < 1 || max_row_len < 1 || topk < 1 || topk > DSA_MAX_TOPK ||
      n_heads < 1)
    return 0;
  if (idx_dtype != DSA_F32 && idx_dtype != DSA_BF16 && idx_dtype != DSA_FP8_E4M3) return 0;
  return prefill_ws(num_rows, num_seqs, max_row_len, idx_dtype, topk, n_heads, dense_threshold);
}

int dsa_sparse_attention_prefill(const dsa_rows *rows, int idx_dtype, int idx_heads, int idx_dim,
                                 const void *q_idx, const float *q_idx_scale, const void *k_idx,
                                 const float *k_idx_scale, const float *w, float *logits,
                                 int64_t ld_logits, int topk, int32_t *idx, int n_heads,
                                 float softmax_scale, const void *q, const void *kv,
                                 const void *w_uk, const void *w_uv, void *out, float *lse,
                                 int dense_threshold, void *ws, size_t ws_bytes, void *stream) {
  return prefill_common(rows, false, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale, k_idx,
                        k_idx_scale, w, logits, ld_logits, topk, idx, n_heads, softmax_scale, q,
                        kv, w_uk, w_uv, out, lse, dense_threshold, ws, ws_bytes, stream);
}

int dsa_sparse_attention_prefill_paged(const dsa_rows *rows, int idx_dtype, int idx_heads,
                                       int idx_dim, const void *q_idx, const float *q_idx_scale,
                                       const void *k_idx, const float *k_idx_scale,
                                       const float *w, float *logits, int64_t ld_logits, int topk,
                                       int32_t *idx, int n_heads, float softmax_scale,
                                       const void *q, const void *kv, const void *w_uk,
                                       const void *w_uv, void *out, float *lse,
                                       int dense_threshold, void *ws, size_t ws_bytes,
                                       void *stream) {
  return prefill_common(rows, true, idx_dtype, idx_heads, idx_dim, q_idx, q_idx_scale, k_idx,
                        k_idx_scale, w, logits, ld_logits, topk, idx, n_heads, softmax_scale, q,
                        kv, w_uk, w_uv, out, lse, dense_threshold, ws, ws_bytes, stream);
}

int dsa_prep_cache_write(int num_tokens, const int32_t *positions, const int64_t *cache_rows,
                         int64_t num_cache_rows, const float *cos_sin, int max_position,
                         int idx_dtype, const void *k_idx_in, void *k_idx_cache,
                         float *k_idx_scale, const void *kv_in, void *kv_cache, void *stream) {
  const dsa::PrepKeys keys{num_tokens, positions, cache_rows, num_cache_rows,
                           k_idx_in, k_idx_cache, k_idx_scale, kv_in, kv_cache};
  const dsa::PrepQueries none{0, nullptr, nullptr, nullptr, nullptr, 1, nullptr};
  return prep_common(keys, none, cos_sin, max_position, idx_dtype, stream);
}

int dsa_prep_queries(int num_rows, const int32_t *positions, const float *cos_sin,
                     int max_position, int idx_dtype, const void *q_idx_in, void *q_idx,
                     float *q_idx_scale, int n_heads, void *q, void *stream) {
  const dsa::PrepKeys none{0, nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, nullptr};
  const dsa::PrepQueries queries{num_rows, positions, q_idx_in, q_idx, q_idx_scale, n_heads, q};
  return prep_common(none, queries, cos_sin, max_position, idx_dtype, stream);
}

int dsa_prep(int num_tokens, const int32_t *positions, const int64_t *cache_rows,
             int64_t num_cache_rows, const float *cos_sin, int max_position, int idx_dtype,
             const void *k_idx_in, void *k_idx_cache, float *k_idx_scale, const void *kv_in,
             void *kv_cache, const void *q_idx_in, void *q_idx, float *q_idx_scale, int n_heads,
             void *q, void *stream) {
  const dsa::PrepKeys keys{num_tokens, positions, cache_rows, num_cache_rows,
                           k_idx_in, k_idx_cache, k_idx_scale, kv_in, kv_cache};
  const dsa::PrepQueries queries{num_tokens, positions, q_idx_in, q_idx, q_idx_scale, n_heads, q};
  return prep_common(keys, queries, cos_sin, max_position, idx_dtype, stream);
}

}  // extern "C"
