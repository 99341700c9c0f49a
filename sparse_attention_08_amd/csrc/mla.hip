// mla.hip -- MLA in MQA mode over the selected cache entries on gfx950.
//
// "DeepSeek-V3.2 技术报告摘要", section 1, MLA-based implementation: DSA runs MLA in
// MQA mode, each latent entry (KV-LoRA latent followed by the RoPE key; "DeepSeek-V3.2
// -- Model techniques map", "Multi-head latent attention") is shared by all query
// heads.  For a row r and head h over the valid selected entries s:
//   z_s = scale * q[r,h,:] . C[s,:] (d_qk = 576),  out[r,h,:] = softmax(z) @ C[:, 0:512]
// with a plain softmax (no sink, no output gate: same page, "Learnable attention sink",
// "Gated attention output").
//
// The bf16 kernels are built from mla_core.h, which describes their design.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "mla_core.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path: one workgroup per (row, head), two passes over the selected entries.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void mla_f32_kernel(RowsDev rows, int H, int Dqk, int Dv,
                                                      float scale, const float *__restrict__ q,
                                                      const float *__restrict__ kv,
                                                      const int32_t *__restrict__ idx, int k,
                                                      float *__restrict__ out,
                                                      float *__restrict__ lse) {
  extern __shared__ float sm[];   // z[k], crow as float bits avoided: separate arrays
  float *z = sm;                                          // [k]
  int64_t *crow = reinterpret_cast<int64_t *>(sm + ((k + 1) & ~1));   // [k]
  float *qs = reinterpret_cast<float *>(crow + k);        // [Dqk]
  __shared__ float red[256 / kWave];
  __shared__ float bcast;
  const int h = blockIdx.x, r = blockIdx.y;
  const int len = rows.row_len[r], b = rows.row_seq[r];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = threadIdx.x; d < Dqk; d += blockDim.x) qs[d] = q[((int64_t)r * H + h) * Dqk + d];
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const int s = idx[(int64_t)r * k + j];
    crow[j] = (s >= 0 && s < len) ? cache_row<PAGED>(rows, b, s) : -1;
  }
  __syncthreads();
  // pass 1: scores and their max
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    float zz = -INFINITY;
    if (crow[j] >= 0) {
      const float *e = kv + crow[j] * Dqk;
      float dot = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(qs[d], e[d], dot);
      zz = dot * scale;
    }
    z[j] = zz;
    mx = fmaxf(mx, zz);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int w = 1; w < (int)(blockDim.x / kWave); ++w) m = fmaxf(m, red[w]);
    bcast = m;
  }
  __syncthreads();
  const float m = bcast;
  // pass 2: weights e^{z-m}, their sum, and the weighted values
  float part = 0.f;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const float p = (crow[j] >= 0) ? expf(z[j] - m) : 0.f;
    z[j] = p;
    part += p;
  }
  part = wave_sum(part);
  __syncthreads();
  if (lane == 0) red[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    float l = 0.f;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) l += red[w];
    bcast = l;
  }
  __syncthreads();
  const float l = bcast;
  for (int d = threadIdx.x; d < Dv; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j)
      if (crow[j] >= 0) acc = fmaf(z[j], kv[crow[j] * Dqk + d], acc);
    out[((int64_t)r * H + h) * Dv + d] = (l > 0.f) ? acc / l : 0.f;
  }
  if (lse && threadIdx.x == 0) lse[(int64_t)r * H + h] = (l > 0.f) ? m + logf(l) : -INFINITY;
}

hipError_t launch_mla_f32(const RowsHost &rh, bool paged, int H, int Dqk, int Dv, float scale,
                          const float *q, const float *kv, const int32_t *idx, int k, float *out,
                          float *lse, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  dim3 grid(H, rh.num_rows);
  const size_t shm = sizeof(float) * ((k + 1) & ~1) + sizeof(int64_t) * k + sizeof(float) * Dqk;
  if (paged)
    mla_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                     lse);
  else
    mla_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                      lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// bf16 MFMA path, d_qk = 576 (512 latent + 64 RoPE), d_v = 512 (mla_core.h)
// ------------------------------------------------------------------------------------
// One workgroup: all 128 heads of query row r over one split of its top-k slots.
// The leading arguments are the ones the prologue needs first (scalars and pointers, so
// the launch can preload them into registers).
template <bool PAGED>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    int R, int splits, int k, int slots_per_split, const int32_t *__restrict__ idx,
    const uint16_t *__restrict__ q, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_len, const int64_t *__restrict__ seq_start,
    const int32_t *__restrict__ page_table, int max_pages, float scale_log2,
    const uint8_t *__restrict__ kv, uint16_t *__restrict__ out, float *__restrict__ lse,
    uint16_t *__restrict__ part_o, float *__restrict__ part_lse) {
  constexpr int H = kHeadsPerBlock;
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_smem[];
  MlaShared &sh = *reinterpret_cast<MlaShared *>(mla_smem);
  MlaCoord co;
  if (!mla_coord(blockIdx.x, R, splits, co)) return;
  const int r = co.r, split = co.split;
  const int slot_begin = split * slots_per_split;
  const int n_slots = max(0, min(k, slot_begin + slots_per_split) - slot_begin);
  const int32_t *idx_row = idx + (int64_t)r * k + slot_begin;
  // the slot loads go out first (they need only the launch arguments), then the query block,
  // then the row's descriptor loads: waits on vector memory are in issue order, so resolving
  // the slots does not wait for the query block (which stays in flight during the slot
  // resolution and the first tile loads)
  int sv[kSlotRounds];
#pragma unroll
  for (int j = 0; j < kSlotRounds; ++j) {
    const int t = j * kMlaThreads + threadIdx.x;
    sv[j] = t < n_slots ? idx_row[t] : -1;
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 qf[18];
  mla_load_q(q, r, qf);
  __builtin_amdgcn_sched_barrier(0);
  const RowsDev rows{row_seq, row_len, seq_start, page_table, max_pages};
  const int n_valid = mla_resolve_slots<PAGED>(sh, sv, n_slots, rows, r);
  // one split: the row's output (natural-log lse); several: the split's partial (log2 lse)
  const bool one = splits == 1;
  const int64_t po = ((int64_t)r * splits + split) * H;
  mla_attend(sh, qf, n_valid, kv, scale_log2, one ? out + (int64_t)r * H * kDv : part_o + po * kDv,
             one ? (lse ? lse + (int64_t)r * H : nullptr) : part_lse + po, one ? kLn2 : 1.f, false);
}

// Merge split partials.  A workgroup of 256 threads merges 4 heads of one row (thread: 8
// dims of one head); workgroups are dealt to XCDs like the split workgroups of their row.
constexpr int kCombHeads = 4;
__global__ __launch_bounds__(256) void mla_combine_kernel(int R, int H, int splits,
                                                          const uint16_t *__restrict__ part_o,
                                                          const float *__restrict__ part_lse,
                                                          uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per_row = H / kCombHeads;
  const int r = (j / per_row) * 8 + x;
  if (r >= R) return;
  const int h = (j % per_row) * kCombHeads + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  mla_combine_head<false>(splits, H, h, d0, part_o + (int64_t)r * splits * H * kDv,
                   part_lse + (int64_t)r * splits * H, out + ((int64_t)r * H + h) * kDv,
                   lse ? lse + (int64_t)r * H + h : nullptr, lse && (threadIdx.x & 63) == 0);
}

#ifndef DSA_MLA_MIN_TILES
#define DSA_MLA_MIN_TILES 4
#endif
int mla_num_splits(int num_rows, int n_heads, int k) {
  // about one workgroup per CU for few-row batches, at least DSA_MLA_MIN_TILES tiles each
  const int base = num_rows * (n_heads / kHeadsPerBlock > 0 ? n_heads / kHeadsPerBlock : 1);
  int splits = (256 + base - 1) / base;
  const int max_splits = (k + DSA_MLA_MIN_TILES * kTile - 1) / (DSA_MLA_MIN_TILES * kTile);
  if (splits > max_splits) splits = max_splits;
  if (splits > kMaxCombine) splits = kMaxCombine;
  if (splits < 1) splits = 1;
  return splits;
}

size_t mla_workspace_bytes(int num_rows, int n_heads, int d_v, int k) {
  const int splits = mla_num_splits(num_rows, n_heads, k);
  if (splits <= 1) return 0;
  // bf16 partial outputs [R, splits, H, d_v], then fp32 partial log-sum-exps [R, splits, H]
  return (size_t)num_rows * splits * n_heads * (sizeof(uint16_t) * (size_t)d_v + sizeof(float));
}

template <bool PAGED>
static hipError_t launch_mla_kernel(unsigned grid, hipStream_t stream, const RowsDev &rows, int R,
                                    float sl2, const uint16_t *q16, const uint8_t *kv8,
                                    const int32_t *idx, int k, int per, int splits, uint16_t *o16,
                                    float *lse, uint16_t *part_o, float *part_lse) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e =
      ensure_dynamic_lds(&mla_bf16_kernel<PAGED>, (int)sizeof(MlaShared), lds_set);
  if (e != hipSuccess) return e;
  mla_bf16_kernel<PAGED><<<grid, kMlaThreads, sizeof(MlaShared), stream>>>(
      R, splits, k, per, idx, q16, rows.row_seq, rows.row_len, rows.seq_start, rows.page_table,
      rows.max_pages, sl2, kv8, o16, lse, part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_mla_bf16(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                           const void *kv, const int32_t *idx, int k, void *out, float *lse,
                           int splits, void *ws, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  const int per = (((k + splits - 1) / splits) + kTile - 1) / kTile * kTile;
  uint16_t *part_o = nullptr;
  float *part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<uint16_t *>(ws);
    part_lse = reinterpret_cast<float *>(part_o + (size_t)rh.num_rows * splits * H * kDv);
  }
  const int R = rh.num_rows;
  const unsigned grid = 8u * (unsigned)((R + 7) / 8) * splits;
  const uint16_t *q16 = static_cast<const uint16_t *>(q);
  const uint8_t *kv8 = static_cast<const uint8_t *>(kv);
  uint16_t *o16 = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  const hipError_t e =
      paged ? launch_mla_kernel<true>(grid, stream, rows, R, sl2, q16, kv8, idx, k, per, splits,
                                      o16, lse, part_o, part_lse)
            : launch_mla_kernel<false>(grid, stream, rows, R, sl2, q16, kv8, idx, k, per, splits,
                                       o16, lse, part_o, part_lse);
  if (e != hipSuccess || splits == 1) return e;
  mla_combine_kernel<<<8u * (unsigned)((R + 7) / 8) * (H / kCombHeads), 256, 0, stream>>>(
      R, H, splits, part_o, part_lse, o16, lse);
  return hipGetLastError();
}

}  // namespace dsa
