// dsa_api.hip -- the C ABI declared in include/dsa.h: argument validation (all of it on
// the host, before anything is enqueued) and dispatch to the kernel launchers.
#include "dsa.h"

#include <math.h>

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

int indexer_common(const dsa_rows *rows, bool paged, int dtype, int n_heads, int head_dim,
                   const void *q, const float *q_scale, const void *k, const float *k_scale,
                   const float *w, float *logits, int64_t ld_logits, void *stream) {
  if (!rows_ok(rows, paged)) return DSA_ERR_INVALID_ARG;
  if (dtype != DSA_F32 && dtype != DSA_BF16 && dtype != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (n_heads <= 0 || head_dim <= 0) return DSA_ERR_INVALID_ARG;
  if (rows->num_rows == 0) return DSA_OK;
  if (!q || !k || !w || !logits) return DSA_ERR_INVALID_ARG;
  if (ld_logits < rows->max_row_len) return DSA_ERR_INVALID_ARG;
  const bool fp8 = dtype == DSA_FP8_E4M3;
  if (fp8 != (q_scale != nullptr) || fp8 != (k_scale != nullptr)) return DSA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const RowsHost rh = to_host(rows);
  if (dtype == DSA_F32) {
    if (n_heads > 64 || head_dim > 256) return DSA_ERR_UNSUPPORTED;
    return status_of(dsa::launch_indexer_f32(rh, paged, n_heads, head_dim,
                                             static_cast<const float *>(q),
                                             static_cast<const float *>(k), w, logits, ld_logits,
                                             s));
  }
  if (n_heads != 64 || head_dim != 128) return DSA_ERR_UNSUPPORTED;
  return status_of(dsa::launch_indexer_mfma(rh, paged, fp8, q, q_scale, k, k_scale, w, logits,
                                            ld_logits, s));
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

int dsa_sparse_mla_prefill(const dsa_rows *rows, int dtype, int n_heads, int d_qk, int d_v,
                           float softmax_scale, const void *q, const void *kv, const int32_t *idx,
                           int k, void *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  return mla_common(rows, false, MlaMode::kPrefill, dtype, n_heads, d_qk, d_v, softmax_scale, q,
                    kv, idx, k, out, lse, nullptr, 0, stream);
}

}  // extern "C"
