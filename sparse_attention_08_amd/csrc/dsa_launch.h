// dsa_launch.h -- host-side launchers of the DSA kernels.  Arguments arrive here
// already validated by the C ABI layer (dsa_api.cpp); these functions only size
// grids and enqueue kernels, and return the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per device (the
// attribute belongs to the device; `done` holds one bit per device id).  Concurrent first
// calls may both set it, which is harmless.
template <class Kernel>
inline hipError_t ensure_dynamic_lds(Kernel *kernel, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Grid of x blocks per row for R rows, rows past the 65535 a grid's y dimension holds
// continuing in z (the kernels recover the row with grid_row()).
constexpr int kMaxGridY = 65535;
inline dim3 row_grid(unsigned x, int R) {
  const unsigned y = R < 1 ? 1u : (R < kMaxGridY ? (unsigned)R : (unsigned)kMaxGridY);
  return dim3(x, y, R < 1 ? 1u : ((unsigned)R + y - 1) / y);
}

struct RowsHost {
  int32_t num_rows;
  int32_t num_seqs;
  const int32_t *row_seq;
  const int32_t *row_len;
  int32_t max_row_len;
  const int64_t *seq_start;
  const int32_t *page_table;
  int32_t max_pages;
};

// ---- indexer ----
hipError_t launch_indexer_f32(const RowsHost &rows, bool paged, int H, int D, const float *q,
                              const float *k, const float *w, float *logits, int64_t ld,
                              hipStream_t stream);
// bf16 / fp8 e4m3 with (H, D) = (64, 128), MFMA path
hipError_t launch_indexer_mfma(const RowsHost &rows, bool paged, bool fp8, const void *q,
                               const float *q_scale, const void *k, const float *k_scale,
                               const float *w, float *logits, int64_t ld, hipStream_t stream);
// bf16, 64 heads x 128 dims, for batches with many rows per sequence (prefill, chunked
// prefill, multi-token decode): workgroups of 8 consecutive rows share each key tile.
hipError_t launch_indexer_prefill(const RowsHost &rows, bool paged, const void *q, const void *k,
                                  const float *w, float *logits, int64_t ld, hipStream_t stream);
// Workgroups per row of the MFMA indexer grid for this batch shape.
int indexer_blocks_per_row(int num_rows, int max_row_len, bool fp8);
// Same, also depositing each workgroup's leading-digit histogram of its scores (the
// first stage of the few-row top-k), indexer_blocks_per_row lists per row.
struct TopkHistDest;
hipError_t launch_indexer_mfma_hist(const RowsHost &rows, bool paged, bool fp8, const void *q,
                                    const float *q_scale, const void *k, const float *k_scale,
                                    const float *w, float *logits, int64_t ld,
                                    const TopkHistDest &hist, hipStream_t stream);

// ---- top-k ----
// Where a producer of scores deposits per-workgroup compressed histograms of the 12-bit
// leading digit of the order keys (list j of row r: count at hcnt[r*stride + j], entries
// (digit << 16 | count) at hlist[(r*stride + j) * 4096 ...]).
struct TopkHistDest {
  uint32_t *hcnt;
  uint32_t *hlist;
  int stride;
};
size_t topk_workspace_bytes(int num_rows, int max_row_len, int k);
// few long rows whose leading-digit histograms come from the score producer
bool topk_hist_fusable(int num_rows, int max_row_len, int hist_lists);
size_t topk_fused_workspace_bytes(int num_rows, int max_row_len, int hist_lists);
TopkHistDest topk_hist_dest(void *ws, int num_rows, int max_row_len, int hist_lists);
hipError_t launch_topk_after_hist(const float *logits, int64_t ld, const int32_t *row_len,
                                  int num_rows, int max_row_len, int k, int32_t *idx, void *ws,
                                  int hist_lists, hipStream_t stream);
// Only the chunk filter of the above: its survivors are left in ws for the attention kernel
// that finishes the selection (launch_mla_bf16_select); rows with row_len <= k are written.
hipError_t launch_topk_filter_after_hist(const float *logits, int64_t ld, const int32_t *row_len,
                                         int num_rows, int max_row_len, int k, int32_t *idx,
                                         void *ws, int hist_lists, hipStream_t stream);
hipError_t launch_topk(const float *logits, int64_t ld, const int32_t *row_len, int num_rows,
                       int max_row_len, int k, int32_t *idx, void *ws, hipStream_t stream);

// ---- sparse MLA ----
int mla_num_splits(int num_rows, int n_heads, int k);
size_t mla_workspace_bytes(int num_rows, int n_heads, int d_v, int k);
hipError_t launch_mla_f32(const RowsHost &rows, bool paged, int H, int Dqk, int Dv, float scale,
                          const float *q, const float *kv, const int32_t *idx, int k, float *out,
                          float *lse, hipStream_t stream);
// bf16 with d_qk = 576, d_v = 512, H % 16 == 0; splits == 1 writes out/lse directly.
hipError_t launch_mla_bf16(const RowsHost &rows, bool paged, int H, float scale, const void *q,
                           const void *kv, const int32_t *idx, int k, void *out, float *lse,
                           int splits, void *ws, hipStream_t stream);
// Same, finishing each row's top-k from the survivors that launch_topk_filter_after_hist left
// in topk_ws (hist_lists as given to it) and writing it to idx.
hipError_t launch_mla_bf16_select(const RowsHost &rows, bool paged, int H, float scale,
                                  const void *q, const void *kv, int32_t *idx, int k, void *out,
                                  float *lse, int splits, void *ws, const float *logits,
                                  int64_t ld, void *topk_ws, int hist_lists, hipStream_t stream);

// ---- masked MHA mode (short prefill) ----
// Workspace: each sequence's reach, its decompressed K_nope and V ([B, max_row_len, H, 128]
// bf16 each) and, with idx, the rows' top-k sets as bit masks.
size_t mha_workspace_bytes(int num_seqs, int H, int R, int max_row_len, bool masked);
// q [R, H, 192] bf16; kv latent cache rows [.., 576] bf16 (only rows the batch reaches are
// read); W_UK, W_UV [H, 128, 512] bf16; idx [R, k] or nullptr (dense causal); out [R, H, 128]
// bf16, lse [R, H] (optional).
// ---- the MQA way of the prefill dispatch (prefill.hip) ----
// q_abs [R, H, 576] = [W_UK[h]^T q_nope | q_rope]; the attention's latent output o_lat
// [R, H, 512] maps back to out [R, H, 128] = W_UV[h] o_lat.
struct AbsorbBuffers {
  uint16_t *wuk_t;   // [H, 512, 128] W_UK transposed
  uint16_t *q_abs;   // [R, H, 576]
  uint16_t *o_lat;   // [R, H, 512]
};
size_t absorb_workspace_bytes(int R, int H);
AbsorbBuffers carve_absorb(void *ws, int R, int H);
hipError_t launch_absorb_query(int R, int H, const void *q, const void *w_uk,
                               const AbsorbBuffers &b, hipStream_t stream);
hipError_t launch_expand_output(int R, int H, const uint16_t *o_lat, const void *w_uv, void *out,
                                hipStream_t stream);

hipError_t launch_mha_prefill(const RowsHost &rows, bool paged, int H, float scale,
                              const void *q, const void *kv, const void *w_uk, const void *w_uv,
                              const int32_t *idx, int k, void *out, float *lse, void *ws,
                              hipStream_t stream);

// ---- indexer-input and cache-write prep ----
// Query rows (R of them, R may be 0): 64 indexer heads rotated to bf16 or e4m3 (+ per-head
// scale), n_heads MLA heads rotated in place.
struct PrepQueries {
  int R;
  const int32_t *pos;
  const void *qi_in;
  void *qi_out;
  float *qi_scale;
  int n_heads;
  void *q;
};
// New tokens (T of them, T may be 0): indexer key (bf16 [T,128]) rotated and written as bf16 or
// e4m3 (+ scale) to cache row rows[t], latent entry (bf16 [T,576]) rotated and written there.
struct PrepKeys {
  int T;
  const int32_t *pos;
  const int64_t *rows;
  int64_t cache_rows;
  const void *k_in;
  void *k_cache;
  float *k_scale;
  const void *kv_in;
  void *kv_cache;
};
// Both sides in one launch.
hipError_t launch_prep(const PrepQueries &queries, const PrepKeys &keys, const float *cos_sin,
                       int max_pos, bool fp8, hipStream_t stream);

}  // namespace dsa
