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
// bf16 kernel design.  A workgroup owns one query row, 64 heads (4 waves x 16 heads)
// and a range of top-k slots.  Selected entries are gathered 32 at a time from HBM with
// 16-byte loads into an LDS tile (double-buffered: the next tile's loads are in flight
// in registers while the current tile is multiplied).  Each wave computes the transposed
// score tile S^T = C . Q^T (keys as MFMA rows, its 16 heads as columns, q resident in
// registers), runs the online softmax in fp32 in the log2 domain, and accumulates
// O += P . V with V read from the same LDS tile through the gfx950 transposing LDS
// read (ds_read_b64_tr_b16), so the tile is stored once, row-major, for both products.
// The LDS tile uses an XOR swizzle of 16-byte chunks so that both the row reads of the
// score product and the transposed reads of the value product are conflict-free.
// Few-row (decode) batches split the slots over several workgroups; each writes a
// normalised partial and its log-sum-exp, and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_launch.h"

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
// bf16 MFMA path, d_qk = 576 (512 latent + 64 RoPE), d_v = 512.
// ------------------------------------------------------------------------------------
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;          // 1152 B per cache entry
constexpr int kChunks = kRowBytes / 16;      // 72 16-byte chunks per entry
constexpr int kTile = 32;                    // entries per LDS tile
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kMlaThreads = 256;             // 4 waves x 16 heads
constexpr int kHeadsPerBlock = 64;
constexpr int kGatherPerThread = kTile * kChunks / kMlaThreads;   // 9
static_assert(kTile * kChunks % kMlaThreads == 0, "gather must split evenly");

// XOR swizzle of the 16-byte chunk index inside its aligned group of 8 chunks.
__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

struct TileMeta {
  int64_t crow[kTile];   // cache row of each tile entry (position 0 of the row's sequence
                         // when the slot is invalid, so loads stay in bounds)
  uint32_t valid;        // bit e set when entry e is a valid selection
};

template <bool PAGED>
__device__ __forceinline__ void tile_meta(TileMeta &m, const RowsDev &rows, int b, int len,
                                          const int32_t *__restrict__ idx_row, int slot0,
                                          int slot_end) {
  // wave 0, lanes 0..31
  const int lane = threadIdx.x;
  const int slot = slot0 + lane;
  int s = -1;
  if (lane < kTile && slot < slot_end) s = idx_row[slot];
  const bool ok = lane < kTile && s >= 0 && s < len;
  const uint64_t vm = __ballot(ok);
  if (lane < kTile) m.crow[lane] = cache_row<PAGED>(rows, b, ok ? s : 0);
  if (lane == 0) m.valid = (uint32_t)vm;
}

__device__ __forceinline__ void gather_issue(i32x4 (&st)[kGatherPerThread], const TileMeta &m,
                                             const uint8_t *__restrict__ kv) {
#pragma unroll
  for (int i = 0; i < kGatherPerThread; ++i) {
    const int j = threadIdx.x + i * kMlaThreads;
    const int e = j / kChunks, ch = j - e * kChunks;
    st[i] = __builtin_nontemporal_load(
        reinterpret_cast<const i32x4 *>(kv + m.crow[e] * kRowBytes) + ch);
  }
}

__device__ __forceinline__ void gather_store(const i32x4 (&st)[kGatherPerThread], uint8_t *tile) {
#pragma unroll
  for (int i = 0; i < kGatherPerThread; ++i) {
    const int j = threadIdx.x + i * kMlaThreads;
    const int e = j / kChunks, ch = j - e * kChunks;
    *reinterpret_cast<i32x4 *>(tile + lds_off(e, ch)) = st[i];
  }
}

typedef bf16x4 __attribute__((address_space(3))) *lds_bf16x4_ptr;

template <bool PAGED>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    RowsDev rows, int H, float scale_log2, const uint16_t *__restrict__ q,
    const uint8_t *__restrict__ kv, const int32_t *__restrict__ idx, int k, int slots_per_split,
    uint16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part_o,
    float *__restrict__ part_lse, int splits) {
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kTileBytes];
  __shared__ TileMeta meta[3];

  const int split = blockIdx.x, hgrp = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r], b = rows.row_seq[r];
  const int h0 = hgrp * kHeadsPerBlock + wave * 16;
  const int slot_begin = split * slots_per_split;
  const int slot_end = min(k, slot_begin + slots_per_split);
  const int n_tiles = slot_end > slot_begin ? (slot_end - slot_begin + kTile - 1) / kTile : 0;
  const int32_t *idx_row = idx + (int64_t)r * k;

  // q^T operand: head h0 + c, dims 32t + 8g .. +8 for t < 18.
  bf16x8 qf[18];
  {
    const bf16x8 *qp =
        reinterpret_cast<const bf16x8 *>(q + ((int64_t)r * H + h0 + c) * kDqk + 8 * g);
#pragma unroll
    for (int t = 0; t < 18; ++t) qf[t] = qp[4 * t];
  }

  f32x4 oacc[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  i32x4 st[kGatherPerThread];
  if (n_tiles > 0) {
    if (wave == 0) tile_meta<PAGED>(meta[0], rows, b, len, idx_row, slot_begin, slot_end);
    __syncthreads();
    if (meta[0].valid) gather_issue(st, meta[0], kv);
    if (wave == 0 && n_tiles > 1)
      tile_meta<PAGED>(meta[1], rows, b, len, idx_row, slot_begin + kTile, slot_end);
    if (meta[0].valid) gather_store(st, tiles[0]);
    __syncthreads();
  }

  // rows of the score tile this lane feeds as the MFMA A operand: two 16-row blocks
  // whose result rows 4g+i map to entries 8g+i and 8g+4+i
  const int arow0 = 8 * (c >> 2) + (c & 3);
  const int arow1 = arow0 + 4;
  const int tr_i = c >> 2, tr_q = c & 3;

  for (int it = 0; it < n_tiles; ++it) {
    const TileMeta &cm = meta[it % 3];
    const bool have_next = it + 1 < n_tiles;
    const TileMeta &nm = meta[(it + 1) % 3];
    if (have_next && nm.valid) gather_issue(st, nm, kv);

    const uint32_t valid = cm.valid;
    if (valid) {
      const uint8_t *tile = tiles[it & 1];
      // ---- scores S^T (entries x heads), K = 576 in 18 steps of 32
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 18; ++t) {
        const int ch = 4 * t + g;
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(tile + lds_off(arow0, ch));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(tile + lds_off(arow1, ch));
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[t], s1, 0, 0, 0);
      }
      // ---- online softmax for head c over entries 8g .. 8g+7 (log2 domain)
      float z[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = ((valid >> (8 * g + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
        z[4 + i] = ((valid >> (8 * g + 4 + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
      }
      float mx = z[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run, mx);          // finite: the tile has a valid entry
      const float alpha = exp2f(m_run - m_new);       // 0 when m_run is -inf
      float p[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2f(z[e] - m_new);
        ps += p[e];
      }
      ps += __shfl_xor(ps, 16, kWave);
      ps += __shfl_xor(ps, 32, kWave);
      l_run = l_run * alpha + ps;
      m_run = m_new;
      // rescale O rows (heads 4g+i) by their head's alpha, only when some max moved
      if (__ballot(alpha != 1.f)) {
        float a4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
        for (int nb = 0; nb < 32; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nb][i] *= a4[i];
      }
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[e];
      // ---- O += P . V, V[entry 8g+e][dv 16nb + c] via two transposing LDS reads
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) {
        const int row_a = 8 * g + tr_i, row_b = row_a + 4;
        const int ch = 2 * nb + (tr_q >> 1);
        const int sub = 8 * (tr_q & 1);
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_ptr)(tile + lds_off(row_a, ch) + sub));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_ptr)(tile + lds_off(row_b, ch) + sub));
        const bf16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vb, oacc[nb], 0, 0, 0);
      }
    }
    if (have_next && nm.valid) gather_store(st, tiles[(it + 1) & 1]);
    if (wave == 0 && it + 2 < n_tiles)
      tile_meta<PAGED>(meta[(it + 2) % 3], rows, b, len, idx_row, slot_begin + (it + 2) * kTile,
                       slot_end);
    __syncthreads();
  }

  // ---- epilogue: heads 4g+i of this wave's 16, dv 16nb + c
  float linv[4], lse2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = __shfl(l_run, 4 * g + i, kWave);
    const float m = __shfl(m_run, 4 * g + i, kWave);
    linv[i] = l > 0.f ? 1.f / l : 0.f;
    lse2[i] = l > 0.f ? m + log2f(l) : -INFINITY;
  }
  if (splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t *op = out + ((int64_t)r * H + h0 + 4 * g + i) * kDv + c;
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) op[16 * nb] = f32_to_bf16_bits(oacc[nb][i] * linv[i]);
      if (lse && c == 0) lse[(int64_t)r * H + h0 + 4 * g + i] = lse2[i] * kLn2;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ph = ((int64_t)r * splits + split) * H + h0 + 4 * g + i;
      float *op = part_o + ph * kDv + c;
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) op[16 * nb] = oacc[nb][i] * linv[i];
      if (c == 0) part_lse[ph] = lse2[i];
    }
  }
}

// Merge split partials: out = sum_s 2^(lse_s - lse) o_s with lse = log2 sum_s 2^lse_s.
__global__ __launch_bounds__(128) void mla_combine_kernel(int H, int splits,
                                                          const float *__restrict__ part_o,
                                                          const float *__restrict__ part_lse,
                                                          uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int h = blockIdx.x, r = blockIdx.y;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, part_lse[((int64_t)r * splits + s) * H + h]);
  float wsum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int d0 = threadIdx.x * 4;
  if (m != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const int64_t ph = ((int64_t)r * splits + s) * H + h;
      const float wgt = exp2f(part_lse[ph] - m);
      wsum += wgt;
      const float4 v = *reinterpret_cast<const float4 *>(part_o + ph * kDv + d0);
      acc[0] = fmaf(wgt, v.x, acc[0]);
      acc[1] = fmaf(wgt, v.y, acc[1]);
      acc[2] = fmaf(wgt, v.z, acc[2]);
      acc[3] = fmaf(wgt, v.w, acc[3]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t *op = out + ((int64_t)r * H + h) * kDv + d0;
#pragma unroll
  for (int j = 0; j < 4; ++j) op[j] = f32_to_bf16_bits(acc[j] * inv);
  if (lse && threadIdx.x == 0)
    lse[(int64_t)r * H + h] = wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

int mla_num_splits(int num_rows, int n_heads, int k) {
  const int base = num_rows * (n_heads / kHeadsPerBlock > 0 ? n_heads / kHeadsPerBlock : 1);
  int splits = (256 + base - 1) / base;
  const int max_splits = (k + 4 * kTile - 1) / (4 * kTile);   // at least 4 tiles per split
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

size_t mla_workspace_bytes(int num_rows, int n_heads, int d_v, int k) {
  const int splits = mla_num_splits(num_rows, n_heads, k);
  if (splits <= 1) return 0;
  return sizeof(float) * (size_t)num_rows * splits * n_heads * ((size_t)d_v + 1);
}

hipError_t launch_mla_bf16(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                           const void *kv, const int32_t *idx, int k, void *out, float *lse,
                           int splits, void *ws, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  const int per = (((k + splits - 1) / splits) + kTile - 1) / kTile * kTile;
  float *part_o = nullptr, *part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<float *>(ws);
    part_lse = part_o + (size_t)rh.num_rows * splits * H * kDv;
  }
  dim3 grid(splits, H / kHeadsPerBlock > 0 ? H / kHeadsPerBlock : 1, rh.num_rows);
  const uint16_t *q16 = static_cast<const uint16_t *>(q);
  const uint8_t *kv8 = static_cast<const uint8_t *>(kv);
  uint16_t *o16 = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  if (paged)
    mla_bf16_kernel<true><<<grid, kMlaThreads, 0, stream>>>(rows, H, sl2, q16, kv8, idx, k, per,
                                                            o16, lse, part_o, part_lse, splits);
  else
    mla_bf16_kernel<false><<<grid, kMlaThreads, 0, stream>>>(rows, H, sl2, q16, kv8, idx, k, per,
                                                             o16, lse, part_o, part_lse, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  mla_combine_kernel<<<dim3(H, rh.num_rows), 128, 0, stream>>>(H, splits, part_o, part_lse, o16,
                                                                lse);
  return hipGetLastError();
}

}  // namespace dsa
