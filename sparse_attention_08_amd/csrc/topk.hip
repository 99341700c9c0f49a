// topk.hip -- fine-grained token selection ("DeepSeek-V3.2 技术报告摘要", section 1,
// DSA ② Fine-grained Token Selection; "DeepSeek-V3.2 -- Model techniques map",
// "Indexer-selected sparse attention": k = min(index_topk, row length), int32 indices).
//
// Exact selection by radix select on order-preserving 32-bit keys: four 8-bit digit
// passes from the most significant end find the key T of the k-th largest score and
// how many of the scores equal to T are still needed; a final ordered pass writes
// every position with key > T plus the lowest-positioned keys == T, in ascending
// position order.  No floating-point arithmetic is involved, so the result is the
// unique set defined by (score desc, position asc) and is bit-exact.
//
// One workgroup per row; when the row fits, it is staged once in LDS and every pass
// reads LDS, otherwise the passes stream the row from L2.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkLdsElems = 32768;   // 128 KB of staged keys

struct TopkShared {
  uint32_t hist[kTopkWaves][256];   // per-wave digit histograms
  uint32_t wave_cnt[2][kTopkWaves];
  uint32_t prefix, mask;
  int32_t need;
};

// Histogram of the digit at `shift` over keys matching (key & mask) == prefix, then the
// digit holding the need-th largest key; updates prefix/mask/need in shared memory.
template <bool STAGED>
__device__ void radix_pass(TopkShared &sh, const uint32_t *keys, const float *row, int n,
                           int shift) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kTopkWaves * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
  __syncthreads();
  const uint32_t prefix = sh.prefix, mask = sh.mask;
  for (int i = threadIdx.x; i < n; i += kTopkThreads) {
    const uint32_t u = STAGED ? keys[i] : order_key(row[i]);
    if ((u & mask) == prefix) atomicAdd(&sh.hist[wave][(u >> shift) & 255u], 1u);
  }
  __syncthreads();
  // fold the per-wave histograms into wave 0's row
  for (int d = threadIdx.x; d < 256; d += kTopkThreads) {
    uint32_t s = 0;
    for (int w = 0; w < kTopkWaves; ++w) s += sh.hist[w][d];
    sh.hist[0][d] = s;
  }
  __syncthreads();
  if (wave == 0) {
    // digits 255..0 in descending order, 4 per lane: lane L owns 255-4L .. 252-4L
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = sh.hist[0][255 - 4 * lane - j];
      tot += c[j];
    }
    // inclusive scan of lane totals (descending digit order)
    uint32_t inc = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    const uint32_t before = inc - tot;   // count of keys in higher digits
    const int32_t need = sh.need;
    // the lane whose range crosses `need`
    if (before < (uint32_t)need && inc >= (uint32_t)need) {
      uint32_t run = before;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run + c[j] >= (uint32_t)need) {
          const uint32_t digit = 255u - 4u * lane - j;
          sh.prefix = prefix | (digit << shift);
          sh.mask = mask | (255u << shift);
          sh.need = need - (int32_t)run;
          break;
        }
        run += c[j];
      }
    }
  }
  __syncthreads();
}

template <bool STAGED>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(const float *__restrict__ logits,
                                                                 int64_t ld,
                                                                 const int32_t *__restrict__ row_len,
                                                                 int k, int32_t *__restrict__ idx) {
  extern __shared__ uint32_t staged[];
  __shared__ TopkShared sh;
  const int r = blockIdx.x;
  const int n = row_len[r];
  const float *row = logits + (int64_t)r * ld;
  int32_t *out = idx + (int64_t)r * k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (n <= k) {   // every position is selected
    for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  if (STAGED) {
    for (int i = threadIdx.x; i < n; i += kTopkThreads) staged[i] = order_key(row[i]);
  }
  if (threadIdx.x == 0) {
    sh.prefix = 0;
    sh.mask = 0;
    sh.need = k;
  }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) radix_pass<STAGED>(sh, staged, row, n, shift);
  const uint32_t T = sh.prefix;      // key of the k-th largest score
  const int32_t need_eq = sh.need;   // how many keys == T to take, lowest positions first

  // Ordered write.  Wave w owns the contiguous span [w*span, (w+1)*span); pass A counts
  // its keys > T and == T, a scan over waves gives each wave its starting ranks, pass B
  // writes in position order with ballot prefix counts.
  const int span = (((n + kTopkWaves - 1) / kTopkWaves) + 63) & ~63;
  const int lo = wave * span;
  const int hi = min(n, lo + span);
  uint32_t gt_cnt = 0, eq_cnt = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    uint32_t u = 0;
    if (i < hi) u = STAGED ? staged[i] : order_key(row[i]);
    gt_cnt += __popcll(__ballot(i < hi && u > T));
    eq_cnt += __popcll(__ballot(i < hi && u == T));
  }
  if (lane == 0) {
    sh.wave_cnt[0][wave] = gt_cnt;
    sh.wave_cnt[1][wave] = eq_cnt;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) eq_before += sh.wave_cnt[1][w];
  for (int w = 0; w < wave; ++w) {
    uint32_t eb = 0;
    for (int v = 0; v < w; ++v) eb += sh.wave_cnt[1][v];
    const int32_t take = max(0, min((int32_t)sh.wave_cnt[1][w], need_eq - (int32_t)eb));
    sel_before += sh.wave_cnt[0][w] + (uint32_t)take;
  }
  const uint64_t lt = lanemask_lt();
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    uint32_t u = 0;
    if (i < hi) u = STAGED ? staged[i] : order_key(row[i]);
    const bool gt = i < hi && u > T;
    const bool eq = i < hi && u == T;
    const uint64_t eq_mask = __ballot(eq);
    const uint32_t eq_rank = eq_before + __popcll(eq_mask & lt);
    const bool sel = gt || (eq && eq_rank < (uint32_t)need_eq);
    const uint64_t sel_mask = __ballot(sel);
    if (sel) out[sel_before + __popcll(sel_mask & lt)] = i;
    eq_before += __popcll(eq_mask);
    sel_before += __popcll(sel_mask);
  }
}

size_t topk_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const float *logits, int64_t ld, const int32_t *row_len, int num_rows,
                       int max_row_len, int k, int32_t *idx, void *, hipStream_t stream) {
  if (max_row_len <= kTopkLdsElems) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_rows_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(sizeof(uint32_t) * kTopkLdsElems));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    topk_rows_kernel<true><<<num_rows, kTopkThreads, sizeof(uint32_t) * max_row_len, stream>>>(
        logits, ld, row_len, k, idx);
  }
  else
    topk_rows_kernel<false><<<num_rows, kTopkThreads, 0, stream>>>(logits, ld, row_len, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
