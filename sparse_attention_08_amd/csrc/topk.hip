// topk.hip -- fine-grained token selection ("DeepSeek-V3.2 技术报告摘要", section 1,
// DSA ② Fine-grained Token Selection; "DeepSeek-V3.2 -- Model techniques map",
// "Indexer-selected sparse attention": k = min(index_topk, row length), int32 indices).
//
// Exact selection on order-preserving 32-bit keys (-0 folded onto +0): a radix select
// with digits of 12, 10 and 10 bits finds the key T of the k-th largest score and how
// many keys equal to T are still needed; an ordered pass then writes every position
// with key > T plus the lowest-positioned keys == T, in ascending position order.  No
// floating-point arithmetic is involved, so the result is the unique set defined by
// (score desc, position asc) and is bit-exact.  The first digit is 12 bits wide (sign,
// exponent and 3 mantissa bits) so that LDS histogram atomics spread over many bins.
//
// Two schedules:
//  * many rows (prefill): one workgroup per row, the row staged once in LDS;
//  * few long rows (decode): each row is cut into 4096-score chunks handled by separate
//    workgroups, in three launches and without device-wide atomics or fences:
//    (1) per chunk, a histogram of the 12-bit digit, stored compressed (nonzero bins);
//    (2) per chunk, every workgroup merges the row's compressed histograms in LDS, finds
//        the digit b* that holds the k-th largest score, and keeps, in position order,
//        the chunk's scores whose digit is >= b* (the k largest are among them);
//    (3) per row, one workgroup gathers those few thousand survivors into LDS and runs
//        the remaining two digits of the exact select on them.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "topk_select.h"

namespace dsa {

#ifndef DSA_TOPK_ROW_THREADS
#define DSA_TOPK_ROW_THREADS 1024   // threads of the one-workgroup-per-row schedule
#endif
constexpr int kSmallThreads = DSA_TOPK_ROW_THREADS;
#ifndef DSA_TOPK_FINAL_THREADS
#define DSA_TOPK_FINAL_THREADS 1024
#endif
constexpr int kFinalThreads = DSA_TOPK_FINAL_THREADS;   // >= kMaxChunks
static_assert(kFinalThreads >= 256 && (1 << 10) % kFinalThreads == 0, "final select shape");
constexpr int kMbThreads = 256;
constexpr int kStageElems = 28672;         // single-row schedule: up to 112 KB of staged keys
static_assert(kStageElems < 65536, "the staged schedule counts its histogram bins in 16 bits");

// ------------------------------------------------------------------------------------
// many-row schedule: one workgroup per row
// ------------------------------------------------------------------------------------
// Rows are taken from the last to the first: in a prefill batch later positions have
// longer rows, so the longest start first and the short ones fill the end of the grid.
// The staged form counts its histogram bins in 16 bits (rows of fewer than 65536 scores),
// so that with rows of up to 16K scores two workgroups share a CU's LDS.
template <bool STAGED>
__global__ __launch_bounds__(kSmallThreads) void topk_row_kernel(const float *__restrict__ logits,
                                                                 int64_t ld,
                                                                 const int32_t *__restrict__ row_len,
                                                                 int k, int32_t *__restrict__ idx) {
  extern __shared__ uint32_t staged[];
  __shared__ BlockScratch<kSmallThreads, STAGED> sh;
  const int r = (int)(gridDim.x - 1 - blockIdx.x);
  const int n = row_len[r];
  const float *row = logits + (int64_t)r * ld;
  int32_t *out = idx + (int64_t)r * k;
  if (n <= k) {
    write_all(out, n, k);
    return;
  }
  if constexpr (STAGED) {
    // the first digit's histogram is counted while the row is staged; every load of a
    // round is issued before any is used
    constexpr int kU = 16;
    for (int i = threadIdx.x; i < kBins / 2; i += kSmallThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
      sh.prefix = 0;
      sh.mask = 0;
      sh.need = k;
    }
    __syncthreads();
    for (int i0 = threadIdx.x; i0 < n; i0 += kU * kSmallThreads) {
      float v[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = i0 + q * kSmallThreads;
        v[q] = i < n ? row[i] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = i0 + q * kSmallThreads;
        if (i < n) {
          const uint32_t u = order_key(v[q]), d = u >> (kD1Bits + kD2Bits);
          staged[i] = u;
          atomicAdd(&sh.hist[d >> 1], 1u << (16 * (d & 1)));
        }
      }
    }
    __syncthreads();
    radix_resolve<kSmallThreads, kD0Bits>(kD1Bits + kD2Bits, sh);
    select_after_first_digit<kSmallThreads>(StagedAcc{staged}, n, out, sh);
  } else {
    select_block<kSmallThreads>(RowAcc{row}, n, k, out, sh);
  }
}

// ------------------------------------------------------------------------------------
// few-row schedule
// ------------------------------------------------------------------------------------
// (1) per-chunk histogram of the 12-bit digit, compressed to its nonzero bins
__global__ __launch_bounds__(kMbThreads) void topk_hist_kernel(const float *__restrict__ logits,
                                                               int64_t ld,
                                                               const int32_t *__restrict__ row_len,
                                                               int k, MbWs ws) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t wtot[kMbThreads / kWave];
  const int r = blockIdx.y, c = blockIdx.x;
  const int n = row_len[r];
  const int base = c * kChunk;
  if (n <= k || base >= n) return;
  const float *row = logits + (int64_t)r * ld;
  for (int i = threadIdx.x; i < kBins; i += kMbThreads) lh[i] = 0;
  __syncthreads();
  {
    // all 16 loads of a thread are issued before any is used
    constexpr int kPerThread = kChunk / kMbThreads;
    float v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = base + threadIdx.x + j * kMbThreads;
      v[j] = i < n ? row[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int i = base + threadIdx.x + j * kMbThreads;
      if (i < n) atomicAdd(&lh[order_key(v[j]) >> (32 - kD0Bits)], 1u);
    }
  }
  __syncthreads();
  // ordered compaction of the nonzero bins: thread t owns bins 16t .. 16t+15
  constexpr int PER = kBins / kMbThreads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t nz = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) nz += lh[PER * threadIdx.x + j] ? 1u : 0u;
  uint32_t inc = wave_incl_scan(nz);
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  uint32_t off = inc - nz, total = 0;
  for (int w = 0; w < kMbThreads / kWave; ++w) {
    off += (w < wave) ? wtot[w] : 0u;
    total += wtot[w];
  }
  uint32_t *dst = ws.hlist + ((size_t)r * ws.C + c) * kBins;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t b = PER * threadIdx.x + j, cnt = lh[b];
    if (cnt) dst[off++] = (b << 16) | cnt;
  }
  if (threadIdx.x == 0) ws.hcnt[(size_t)r * ws.C + c] = total;
}

// (2) merge the row's histograms, find b*, keep this chunk's survivors in position order.
// One round of independent loads: the chunk's scores, then every histogram list's count
// together with its first entries (a list is read by several threads); only lists longer
// than that need a second round.
__global__ __launch_bounds__(kMbThreads) void topk_filter_kernel(const float *__restrict__ logits,
                                                                 int64_t ld,
                                                                 const int32_t *__restrict__ row_len,
                                                                 int k, int32_t *__restrict__ idx,
                                                                 MbWs ws) {
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t wtot[kMbThreads / kWave];
  __shared__ uint32_t wcnt[kMbThreads / kWave];
  __shared__ uint32_t s_bstar, s_above;
  const int r = blockIdx.y, c = blockIdx.x;
  const int n = row_len[r];
  const int base = c * kChunk;
  if (n <= k) {
    if (c == 0) write_all(idx + (int64_t)r * k, n, k);
    return;
  }
  if (base >= n) return;
  const int nblk = (n + kChunk - 1) / kChunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // this chunk's scores (wave w owns 1024 consecutive positions)
  const float *row = logits + (int64_t)r * ld;
  constexpr int kPerWave = kChunk / (kMbThreads / kWave);   // 1024 scores per wave
  constexpr int kIter = kPerWave / 64;
  const int wlo = base + wave * kPerWave;
  float sv[kIter];
#pragma unroll
  for (int j = 0; j < kIter; ++j) {
    const int i = wlo + 64 * j + lane;
    sv[j] = i < n ? row[i] : 0.f;
  }
  // every histogram list of the row: tpl threads per list (nh <= kMaxChunks = kMbThreads)
  const int nh = ws.nh ? ws.nh : nblk;
  int tpl = kMbThreads;
  while (tpl > 1 && tpl * nh > kMbThreads) tpl >>= 1;
  const int l = threadIdx.x / tpl, sub = threadIdx.x % tpl;
  const uint32_t *hl = ws.hlist + ((size_t)r * ws.C + l) * kBins;
  uint32_t cnt = 0, ent[kListHead];
  if (l < nh) {
    cnt = ws.hcnt[(size_t)r * ws.C + l];
#pragma unroll
    for (int j = 0; j < kListHead; ++j) ent[j] = hl[sub + tpl * j];   // within the list's bins
  }
  for (int i = threadIdx.x; i < kBins; i += kMbThreads) lh[i] = 0;
  __syncthreads();
  if (l < nh) {
#pragma unroll
    for (int j = 0; j < kListHead; ++j)
      if ((uint32_t)(sub + tpl * j) < cnt) atomicAdd(&lh[ent[j] >> 16], ent[j] & 0xFFFFu);
    for (uint32_t e = tpl * kListHead + sub; e < cnt; e += tpl) {
      const uint32_t v = hl[e];
      atomicAdd(&lh[v >> 16], v & 0xFFFFu);
    }
  }
  __syncthreads();
  // digit b* holding the k-th largest: thread t owns bins 4095-16t-j (descending)
  constexpr int PER = kBins / kMbThreads;
  uint32_t cc[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    cc[j] = lh[kBins - 1 - PER * threadIdx.x - j];
    tot += cc[j];
  }
  uint32_t inc = wave_incl_scan(tot);
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  uint32_t before = inc - tot;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  if (before < (uint32_t)k && before + tot >= (uint32_t)k) {
    uint32_t run = before;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (run + cc[j] >= (uint32_t)k) {
        s_bstar = kBins - 1 - PER * threadIdx.x - j;
        s_above = run;
        break;
      }
      run += cc[j];
    }
  }
  __syncthreads();
  const uint32_t bstar = s_bstar;
  if (c == 0 && threadIdx.x == 0) {
    ws.meta[2 * r] = bstar;
    ws.meta[2 * r + 1] = s_above;
  }
  // survivors of this chunk (digit >= b*), in position order
  uint32_t keys[kIter];
  uint32_t wc = 0;
#pragma unroll
  for (int j = 0; j < kIter; ++j) {
    const int i = wlo + 64 * j + lane;
    keys[j] = order_key(sv[j]);
    wc += __popcll(__ballot(i < n && (keys[j] >> (32 - kD0Bits)) >= bstar));
  }
  if (lane == 0) wcnt[wave] = wc;
  __syncthreads();
  uint32_t soff = 0, stotal = 0;
  for (int w = 0; w < kMbThreads / kWave; ++w) {
    soff += (w < wave) ? wcnt[w] : 0u;
    stotal += wcnt[w];
  }
  uint2 *lst = ws.slist + ((size_t)r * ws.C + c) * kChunk;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int j = 0; j < kIter; ++j) {
    const int i = wlo + 64 * j + lane;
    const bool keep = i < n && (keys[j] >> (32 - kD0Bits)) >= bstar;
    const uint64_t m = __ballot(keep);
    if (keep) lst[soff + __popcll(m & lt)] = make_uint2(keys[j], (uint32_t)i);
    soff += __popcll(m);
  }
  if (threadIdx.x == 0) ws.scnt[(size_t)r * ws.C + c] = stotal;
}

// (3) one workgroup per row: exact select among the survivors, gathered with the chunk
// counts in one round of loads
template <int NT>
__global__ __launch_bounds__(NT) void topk_final_kernel(const float *__restrict__ logits,
                                                        int64_t ld,
                                                        const int32_t *__restrict__ row_len,
                                                        int k, int32_t *__restrict__ idx,
                                                        MbWs ws) {
  __shared__ BlockScratch<NT> sh;
  __shared__ uint32_t skey[kSurvivorCap];
  __shared__ int32_t spos[kSurvivorCap];
  __shared__ uint32_t coff[kMaxChunks + 1];
  const int r = blockIdx.x;
  const int n = row_len[r];
  if (n <= k) return;
  const SurvivorLoads<NT> L = issue_survivor_loads<NT>(ws, r, (n + kChunk - 1) / kChunk);
  select_from_survivors<NT>(L, logits, ld, ws, r, n, k, idx + (int64_t)r * k, sh, skey, spos, coff);
}

// ------------------------------------------------------------------------------------
// dispatch
// ------------------------------------------------------------------------------------
static bool few_rows(int num_rows, int max_row_len) {
  // Long rows that cannot fill the GPU with one workgroup each go to the chunked schedule.
  return max_row_len > 8192 && num_rows < 256 && max_row_len <= kMaxChunks * kChunk;
}

size_t topk_workspace_bytes(int num_rows, int max_row_len, int) {
  if (!few_rows(num_rows, max_row_len)) return 0;
  const int C = (max_row_len + kChunk - 1) / kChunk;
  return mb_ws_bytes(num_rows, C);
}

bool topk_hist_fusable(int num_rows, int max_row_len, int hist_lists) {
  return few_rows(num_rows, max_row_len) && hist_lists >= 1 && hist_lists <= kMaxChunks;
}

size_t topk_fused_workspace_bytes(int num_rows, int max_row_len, int hist_lists) {
  const int C = (max_row_len + kChunk - 1) / kChunk;
  return mb_ws_bytes(num_rows, C > hist_lists ? C : hist_lists);
}

TopkHistDest topk_hist_dest(void *ws, int num_rows, int max_row_len, int hist_lists) {
  const int C = (max_row_len + kChunk - 1) / kChunk;
  const MbWs w = carve_ws(ws, num_rows, C > hist_lists ? C : hist_lists);
  return TopkHistDest{w.hcnt, w.hlist, w.C};
}

hipError_t launch_topk_filter_after_hist(const float *logits, int64_t ld, const int32_t *row_len,
                                         int num_rows, int max_row_len, int k, int32_t *idx,
                                         void *ws, int hist_lists, hipStream_t stream) {
  const MbWs w = topk_chunk_ws(ws, num_rows, max_row_len, hist_lists);
  dim3 grid((max_row_len + kChunk - 1) / kChunk, num_rows);
  topk_filter_kernel<<<grid, kMbThreads, 0, stream>>>(logits, ld, row_len, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_topk_after_hist(const float *logits, int64_t ld, const int32_t *row_len,
                                  int num_rows, int max_row_len, int k, int32_t *idx, void *ws,
                                  int hist_lists, hipStream_t stream) {
  hipError_t e = launch_topk_filter_after_hist(logits, ld, row_len, num_rows, max_row_len, k, idx,
                                               ws, hist_lists, stream);
  if (e != hipSuccess) return e;
  const MbWs w = topk_chunk_ws(ws, num_rows, max_row_len, hist_lists);
  topk_final_kernel<kFinalThreads><<<num_rows, kFinalThreads, 0, stream>>>(logits, ld, row_len, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int64_t ld, const int32_t *row_len, int num_rows,
                       int max_row_len, int k, int32_t *idx, void *ws, hipStream_t stream) {
  if (few_rows(num_rows, max_row_len)) {
    const int C = (max_row_len + kChunk - 1) / kChunk;
    const MbWs w = carve_ws(ws, num_rows, C);
    dim3 grid(C, num_rows);
    topk_hist_kernel<<<grid, kMbThreads, 0, stream>>>(logits, ld, row_len, k, w);
    topk_filter_kernel<<<grid, kMbThreads, 0, stream>>>(logits, ld, row_len, k, idx, w);
    topk_final_kernel<kFinalThreads><<<num_rows, kFinalThreads, 0, stream>>>(logits, ld, row_len, k, idx, w);
    return hipGetLastError();
  }
  if (max_row_len <= kStageElems) {
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e = ensure_dynamic_lds(&topk_row_kernel<true>,
                                            (int)(sizeof(uint32_t) * kStageElems), lds_set);
    if (e != hipSuccess) return e;
    topk_row_kernel<true><<<num_rows, kSmallThreads, sizeof(uint32_t) * max_row_len, stream>>>(
        logits, ld, row_len, k, idx);
  } else {
    topk_row_kernel<false><<<num_rows, kSmallThreads, 0, stream>>>(logits, ld, row_len, k, idx);
  }
  return hipGetLastError();
}

}  // namespace dsa
