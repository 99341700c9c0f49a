// indexer.hip -- lightning-indexer scores on gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:]) over the preceding tokens s of the
// query's sequence ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ① Lightning Indexer:
// a few indexer heads, one key per token shared by all heads, FP8 supported).
//
// Decode-shaped work (few query rows, long contexts) is bound by the key stream from
// HBM: every key byte is read once and meets 64 heads (64 flop/B in bf16, 128 flop/B
// in fp8), far under the MFMA ridge.  The MFMA kernel therefore gives each wave a
// contiguous span of keys, keeps the row's 64x128 query block resident in registers as
// MFMA operands, streams keys straight from HBM into registers (no LDS round trip,
// the next key group is in flight while the current one is multiplied), and fuses
// ReLU, the head weights, the fp8 scales and the 64-head sum into the MFMA epilogue.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path (any small H, D): one thread per key, plain fp32 FMA.  This is the
// exactness path (checked at 1e-5 relative) and is not tuned.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void indexer_f32_kernel(RowsDev rows, int H, int D,
                                                          const float *__restrict__ q,
                                                          const float *__restrict__ k,
                                                          const float *__restrict__ w,
                                                          float *__restrict__ logits, int64_t ld) {
  extern __shared__ float smem[];   // q row [H*D] then w row [H]
  const int r = blockIdx.y;
  const int len = rows.row_len[r];
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((int64_t)blockIdx.x * blockDim.x >= len) return;
  float *qs = smem;
  float *ws = smem + H * D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) qs[i] = q[(int64_t)r * H * D + i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) ws[i] = w[(int64_t)r * H + i];
  __syncthreads();
  if (s >= len) return;
  const int b = rows.row_seq[r];
  const float *kr = k + cache_row<PAGED>(rows, b, s) * D;
  float acc = 0.f;
  for (int j = 0; j < H; ++j) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qs[j * D + d], kr[d], dot);
    acc = fmaf(ws[j], fmaxf(dot, 0.f), acc);
  }
  logits[(int64_t)r * ld + s] = acc;
}

hipError_t launch_indexer_f32(const RowsHost &rh, bool paged, int H, int D, const float *q,
                              const float *k, const float *w, float *logits, int64_t ld,
                              hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  dim3 grid((rh.max_row_len + 255) / 256, rh.num_rows);
  size_t shm = sizeof(float) * ((size_t)H * D + H);
  if (paged)
    indexer_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, H, D, q, k, w, logits, ld);
  else
    indexer_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, H, D, q, k, w, logits, ld);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// MFMA path, 64 heads x 128 dims, bf16 or OCP e4m3.
//
// Per wave, a 16-key tile is the N dimension of a 16x16 MFMA tile, 16 heads the M
// dimension (4 head blocks cover 64 heads) and the 128 dims the K dimension.  Lane
// (g = lane/16, c = lane%16) holds, for its key c, dims [32g, 32g+32) as the B operand
// and, for head 16*hb + c, the same dims of q as the A operand; the result lane holds
// heads 16*hb + 4g + i (i < 4) of key c.  Since A and B use the same dim->slot map, the
// contraction is the plain dot product.
//   bf16: 4 x v_mfma_f32_16x16x32_bf16 per head block (K = 32 each)
//   fp8 : 1 x v_mfma_scale_f32_16x16x128_f8f6f4 per head block (K = 128, unit scales)
// Epilogue per key: v = sum_{hb,i} w'[head] * max(acc, 0) over the lane's 16 heads,
// then a 4-lane sum across g; fp8 multiplies by the key's scale, and w' = w * q_scale.
// ------------------------------------------------------------------------------------
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;

template <bool FP8>
struct KeyFrag {
  static constexpr int kChunks = FP8 ? 2 : 4;   // 16-byte chunks a lane loads per key
  i32x4 c[kChunks];
};

template <bool FP8, bool PAGED>
__device__ __forceinline__ void load_key(KeyFrag<FP8> &f, float &ks, const uint8_t *__restrict__ k,
                                         const float *__restrict__ k_scale, const RowsDev &rows,
                                         int b, int64_t s, int g) {
  constexpr int kRowBytes = kIdxDim * (FP8 ? 1 : 2);
  const int64_t crow = cache_row<PAGED>(rows, b, s);
  const i32x4 *p = reinterpret_cast<const i32x4 *>(k + crow * kRowBytes + g * (kRowBytes / 4));
#pragma unroll
  for (int i = 0; i < KeyFrag<FP8>::kChunks; ++i) f.c[i] = __builtin_nontemporal_load(p + i);
  if constexpr (FP8) ks = k_scale[crow];
}

template <bool FP8, bool PAGED, int U>
__global__ __launch_bounds__(256) void indexer_mfma_kernel(
    RowsDev rows, const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, const float *__restrict__ w,
    float *__restrict__ logits, int64_t ld, int keys_per_wave) {
  constexpr int kElt = FP8 ? 1 : 2;
  constexpr int kRowBytes = kIdxDim * kElt;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r];
  const int64_t s_begin = ((int64_t)blockIdx.x * 4 + wave) * keys_per_wave;
  if (s_begin >= len) return;
  const int64_t s_end = min<int64_t>(s_begin + keys_per_wave, len);
  const int b = rows.row_seq[r];

  // Query operand: head 16*hb + c, dims [32g, 32g+32).
  i32x4 qf[4][KeyFrag<FP8>::kChunks];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const i32x4 *p = reinterpret_cast<const i32x4 *>(
        q + ((int64_t)r * kIdxHeads + hb * 16 + c) * kRowBytes + g * (kRowBytes / 4));
#pragma unroll
    for (int i = 0; i < KeyFrag<FP8>::kChunks; ++i) qf[hb][i] = p[i];
  }
  // Head weights for the result rows this lane holds: heads 16*hb + 4g + i.
  float wt[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t hj = (int64_t)r * kIdxHeads + hb * 16 + 4 * g + i;
      wt[hb][i] = FP8 ? w[hj] * q_scale[hj] : w[hj];
    }

  KeyFrag<FP8> cur[U], nxt[U];
  float cur_s[U], nxt_s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t s = min<int64_t>(s_begin + 16 * u + c, s_end - 1);
    load_key<FP8, PAGED>(cur[u], cur_s[u], k, k_scale, rows, b, s, g);
  }
  float *out = logits + (int64_t)r * ld;
  for (int64_t s0 = s_begin; s0 < s_end; s0 += 16 * U) {
    const bool more = s0 + 16 * U < s_end;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t s = min<int64_t>(s0 + 16 * U + 16 * u + c, s_end - 1);
        load_key<FP8, PAGED>(nxt[u], nxt_s[u], k, k_scale, rows, b, s, g);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 acc[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
          const i32x8 a = __builtin_shufflevector(qf[hb][0], qf[hb][1], 0, 1, 2, 3, 4, 5, 6, 7);
          const i32x8 bb =
              __builtin_shufflevector(cur[u].c[0], cur[u].c[1], 0, 1, 2, 3, 4, 5, 6, 7);
          acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, acc[hb], 0, 0, 0, 127,
                                                                     0, 127);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, qf[hb][t]), __builtin_bit_cast(bf16x8, cur[u].c[t]),
                acc[hb], 0, 0, 0);
        }
      }
      float v = 0.f;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(wt[hb][i], fmaxf(acc[hb][i], 0.f), v);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      if constexpr (FP8) v *= cur_s[u];
      const int64_t s = s0 + 16 * u + c;
      if (g == 0 && s < s_end) out[s] = v;
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cur[u] = nxt[u];
        cur_s[u] = nxt_s[u];
      }
    }
  }
}

hipError_t launch_indexer_mfma(const RowsHost &rh, bool paged, bool fp8, const void *q,
                               const float *q_scale, const void *k, const float *k_scale,
                               const float *w, float *logits, int64_t ld, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  // Aim for ~4096+ waves (16 per CU on 256 CUs); spans are whole 16-key tiles.
  const int64_t total = (int64_t)rh.num_rows * rh.max_row_len;
  int64_t kpw = (total + 8191) / 8192;
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  if (kpw > 2048) kpw = 2048;
  const int64_t per_block = 4 * kpw;
  dim3 grid((unsigned)((rh.max_row_len + per_block - 1) / per_block), rh.num_rows);
  const uint8_t *q8 = static_cast<const uint8_t *>(q);
  const uint8_t *k8 = static_cast<const uint8_t *>(k);
  if (fp8) {
    if (paged)
      indexer_mfma_kernel<true, true, 4><<<grid, 256, 0, stream>>>(rows, q8, q_scale, k8, k_scale,
                                                                   w, logits, ld, (int)kpw);
    else
      indexer_mfma_kernel<true, false, 4><<<grid, 256, 0, stream>>>(rows, q8, q_scale, k8, k_scale,
                                                                    w, logits, ld, (int)kpw);
  } else {
    if (paged)
      indexer_mfma_kernel<false, true, 2><<<grid, 256, 0, stream>>>(rows, q8, q_scale, k8, k_scale,
                                                                    w, logits, ld, (int)kpw);
    else
      indexer_mfma_kernel<false, false, 2><<<grid, 256, 0, stream>>>(rows, q8, q_scale, k8,
                                                                     k_scale, w, logits, ld,
                                                                     (int)kpw);
  }
  return hipGetLastError();
}

}  // namespace dsa
