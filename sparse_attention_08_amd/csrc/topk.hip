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

namespace dsa {

constexpr int kD0Bits = kLeadDigitBits, kD1Bits = 10, kD2Bits = 10;
constexpr int kBins = 1 << kD0Bits;        // 4096
constexpr int kChunk = 4096;               // scores per workgroup in the few-row schedule
constexpr int kSmallThreads = 1024;
#ifndef DSA_TOPK_FINAL_THREADS
#define DSA_TOPK_FINAL_THREADS 1024
#endif
constexpr int kFinalThreads = DSA_TOPK_FINAL_THREADS;   // >= kMaxChunks
static_assert(kFinalThreads >= 256 && (1 << 10) % kFinalThreads == 0, "final select shape");
constexpr int kMbThreads = 256;
constexpr int kStageElems = 28672;         // single-row schedule: up to 112 KB of staged keys
constexpr int kSurvivorCap = 10240;        // survivors selected in LDS (80 KB)
constexpr int kMaxChunks = 256;            // chunked schedule handles rows up to 1M scores
constexpr int kListHead = 8;               // histogram entries per thread loaded with the counts
constexpr int kSurvHead = 4;               // survivors per thread loaded with the chunk counts

// ------------------------------------------------------------------------------------
// block-wide helpers
// ------------------------------------------------------------------------------------
template <int NT>
struct BlockScratch {
  uint32_t hist[kBins];
  uint32_t wsum[NT / kWave];
  uint32_t wcnt[2][NT / kWave];
  uint32_t prefix, mask;
  int32_t need;
  uint32_t flag;
};

// Exclusive prefix sum over the block's threads of v; returns it and the block total.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total,
                                                    BlockScratch<NT> &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == 63) sh.wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t s = sh.wsum[w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// One radix digit: histogram of digit (key >> shift) & (2^BITS - 1) over the keys that
// match (key & mask) == prefix, then the digit holding the need-th largest key.
template <int NT, int BITS, class Acc>
__device__ void radix_digit(const Acc &acc, int n, int shift, BlockScratch<NT> &sh) {
  constexpr int NB = 1 << BITS;
  constexpr int PER = NB / NT;             // consecutive bins owned per thread
  static_assert(NB % NT == 0, "bins must split evenly");
  for (int i = threadIdx.x; i < NB; i += NT) sh.hist[i] = 0;
  __syncthreads();
  const uint32_t prefix = sh.prefix, mask = sh.mask;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t u = acc.key(i);
    if ((u & mask) == prefix) atomicAdd(&sh.hist[(u >> shift) & (NB - 1)], 1u);
  }
  __syncthreads();
  // thread t owns bins NB-1-PER*t-j (j < PER): descending digit order across threads
  uint32_t c[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    c[j] = sh.hist[NB - 1 - PER * threadIdx.x - j];
    tot += c[j];
  }
  uint32_t all;
  const uint32_t before = block_excl_scan<NT>(tot, all, sh);
  const int32_t need = sh.need;
  __syncthreads();
  if (before < (uint32_t)need && before + tot >= (uint32_t)need) {
    uint32_t run = before;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (run + c[j] >= (uint32_t)need) {
        const uint32_t digit = NB - 1 - PER * threadIdx.x - j;
        sh.prefix = prefix | (digit << shift);
        sh.mask = mask | ((uint32_t)(NB - 1) << shift);
        sh.need = need - (int32_t)run;
        break;
      }
      run += c[j];
    }
  }
  __syncthreads();
}

// Exact top-k of n keys given by acc (key(i), pos(i); items in ascending position
// order), written to out[0..k) in ascending position order.  Requires n > k.
// When first_digit >= 0 the caller already knows the 12-bit digit of T and that
// `need_in_digit` keys with that digit belong to the result.
template <int NT, class Acc>
__device__ void select_block(const Acc &acc, int n, int k, int32_t *__restrict__ out,
                             BlockScratch<NT> &sh, int first_digit = -1, int need_in_digit = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    if (first_digit >= 0) {
      sh.prefix = (uint32_t)first_digit << (kD1Bits + kD2Bits);
      sh.mask = (uint32_t)(kBins - 1) << (kD1Bits + kD2Bits);
      sh.need = need_in_digit;
    } else {
      sh.prefix = 0;
      sh.mask = 0;
      sh.need = k;
    }
  }
  __syncthreads();
  if (first_digit < 0) radix_digit<NT, kD0Bits>(acc, n, kD1Bits + kD2Bits, sh);
  radix_digit<NT, kD1Bits>(acc, n, kD2Bits, sh);
  radix_digit<NT, kD2Bits>(acc, n, 0, sh);
  const uint32_t T = sh.prefix;
  const int32_t need_eq = sh.need;
  // ordered write: wave w owns a contiguous span; counts, wave offsets, then ballots
  constexpr int NW = NT / kWave;
  const int span = (((n + NW - 1) / NW) + 63) & ~63;
  const int lo = wave * span, hi = min(n, lo + span);
  uint32_t gt_cnt = 0, eq_cnt = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t u = i < hi ? acc.key(i) : 0u;
    gt_cnt += __popcll(__ballot(i < hi && u > T));
    eq_cnt += __popcll(__ballot(i < hi && u == T));
  }
  if (lane == 0) {
    sh.wcnt[0][wave] = gt_cnt;
    sh.wcnt[1][wave] = eq_cnt;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int32_t take = max(0, min((int32_t)sh.wcnt[1][w], need_eq - (int32_t)eq_before));
    sel_before += sh.wcnt[0][w] + (uint32_t)take;
    eq_before += sh.wcnt[1][w];
  }
  const uint64_t lt = lanemask_lt();
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const uint32_t u = i < hi ? acc.key(i) : 0u;
    const bool gt = i < hi && u > T;
    const bool eq = i < hi && u == T;
    const uint64_t eq_mask = __ballot(eq);
    const uint32_t eq_rank = eq_before + __popcll(eq_mask & lt);
    const bool sel = gt || (eq && eq_rank < (uint32_t)need_eq);
    const uint64_t sel_mask = __ballot(sel);
    if (sel) out[sel_before + __popcll(sel_mask & lt)] = acc.pos(i);
    eq_before += __popcll(eq_mask);
    sel_before += __popcll(sel_mask);
  }
}

struct RowAcc {            // keys computed on the fly from a score row in global memory
  const float *row;
  __device__ uint32_t key(int i) const { return order_key(row[i]); }
  __device__ int32_t pos(int i) const { return i; }
};
struct StagedAcc {         // keys staged in LDS
  const uint32_t *keys;
  __device__ uint32_t key(int i) const { return keys[i]; }
  __device__ int32_t pos(int i) const { return i; }
};
struct SurvivorAcc {       // (key, position) survivors staged in LDS
  const uint32_t *keys;
  const int32_t *posn;
  __device__ uint32_t key(int i) const { return keys[i]; }
  __device__ int32_t pos(int i) const { return posn[i]; }
};

__device__ __forceinline__ void write_all(int32_t *out, int n, int k) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < n ? i : -1;
}

// ------------------------------------------------------------------------------------
// many-row schedule: one workgroup per row
// ------------------------------------------------------------------------------------
template <bool STAGED>
__global__ __launch_bounds__(kSmallThreads) void topk_row_kernel(const float *__restrict__ logits,
                                                                 int64_t ld,
                                                                 const int32_t *__restrict__ row_len,
                                                                 int k, int32_t *__restrict__ idx) {
  extern __shared__ uint32_t staged[];
  __shared__ BlockScratch<kSmallThreads> sh;
  const int r = blockIdx.x;
  const int n = row_len[r];
  const float *row = logits + (int64_t)r * ld;
  int32_t *out = idx + (int64_t)r * k;
  if (n <= k) {
    write_all(out, n, k);
    return;
  }
  if constexpr (STAGED) {
    for (int i = threadIdx.x; i < n; i += kSmallThreads) staged[i] = order_key(row[i]);
    __syncthreads();
    select_block<kSmallThreads>(StagedAcc{staged}, n, k, out, sh);
  } else {
    select_block<kSmallThreads>(RowAcc{row}, n, k, out, sh);
  }
}

// ------------------------------------------------------------------------------------
// few-row schedule
// ------------------------------------------------------------------------------------
struct MbWs {
  uint32_t *hcnt;     // [R][C]          nonzero bins per chunk histogram
  uint32_t *hlist;    // [R][C][kBins]   (digit << 16 | count) of the nonzero bins
  uint32_t *meta;     // [R][2]          b*, number of scores with digit > b*
  uint32_t *scnt;     // [R][C]          survivors per chunk
  uint2 *slist;       // [R][C][kChunk]  (key, position) survivors per chunk
  int C;              // chunk stride of the arrays above
  int nh;             // histogram lists per row; 0: one per 4096-score chunk of the row
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t mb_ws_bytes(int R, int C) {
  return align256(sizeof(uint32_t) * (size_t)R * C) * 2 +
         align256(sizeof(uint32_t) * (size_t)R * C * kBins) + align256(sizeof(uint32_t) * (size_t)R * 2) +
         sizeof(uint2) * (size_t)R * C * kChunk;
}

__host__ __device__ inline MbWs carve_ws(void *ws, int R, int C) {
  uint8_t *p = static_cast<uint8_t *>(ws);
  MbWs w;
  w.hcnt = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * C);
  w.scnt = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * C);
  w.hlist = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * C * kBins);
  w.meta = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * 2);
  w.slist = reinterpret_cast<uint2 *>(p);
  w.C = C;
  w.nh = 0;
  return w;
}

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
  uint32_t inc = nz;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
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

// Chunk j of the flattened list whose exclusive prefix offsets are off[0..nc] (off[nc] =
// total): the last j with off[j] <= e.  Binary search over LDS.
__device__ __forceinline__ int chunk_of(const uint32_t *off, int nc, uint32_t e) {
  int lo = 0, hi = nc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  return lo;
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
  uint32_t inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
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

// (3) one workgroup per row: exact select among the survivors, gathered with independent
// loads (chunk of each survivor found from the prefix of the per-chunk counts)
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
  int32_t *out = idx + (int64_t)r * k;
  const int nblk = (n + kChunk - 1) / kChunk;
  const int bstar = (int)ws.meta[2 * r];
  const int above = (int)ws.meta[2 * r + 1];
  // survivor counts of the chunks and each chunk's first survivors in one round of loads:
  // tpc threads per chunk (nblk <= kMaxChunks <= NT), kSurvHead survivors each
  int tpc = NT;
  while (tpc > 1 && tpc * nblk > NT) tpc >>= 1;
  const int ch = threadIdx.x / tpc, sub = threadIdx.x % tpc;
  const uint2 *cl = ws.slist + ((size_t)r * ws.C + ch) * kChunk;
  uint32_t cnt = 0;
  uint2 head[kSurvHead];
  if (ch < nblk) {
    cnt = ws.scnt[(size_t)r * ws.C + ch];
#pragma unroll
    for (int j = 0; j < kSurvHead; ++j) head[j] = cl[sub + tpc * j];   // within the chunk's list
  }
  {
    uint32_t total;
    const uint32_t before = block_excl_scan<NT>(sub == 0 ? cnt : 0u, total, sh);
    if (sub == 0 && ch < nblk) coff[ch] = before;
    if (threadIdx.x == 0) coff[nblk] = total;
  }
  __syncthreads();
  const int M = (int)coff[nblk];
  if (M <= kSurvivorCap) {
    if (ch < nblk) {
      const int dst = (int)coff[ch];
#pragma unroll
      for (int j = 0; j < kSurvHead; ++j) {
        const uint32_t e = sub + tpc * j;
        if (e < cnt) {
          skey[dst + e] = head[j].x;
          spos[dst + e] = (int32_t)head[j].y;
        }
      }
      for (uint32_t e = tpc * kSurvHead + sub; e < cnt; e += tpc) {
        const uint2 v = cl[e];
        skey[dst + e] = v.x;
        spos[dst + e] = (int32_t)v.y;
      }
    }
    __syncthreads();
    select_block<NT>(SurvivorAcc{skey, spos}, M, k, out, sh, bstar, k - above);
  } else {
    // degenerate score distributions (huge ties around the threshold): whole row
    select_block<NT>(RowAcc{logits + (int64_t)r * ld}, n, k, out, sh, bstar, k - above);
  }
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

hipError_t launch_topk_after_hist(const float *logits, int64_t ld, const int32_t *row_len,
                                  int num_rows, int max_row_len, int k, int32_t *idx, void *ws,
                                  int hist_lists, hipStream_t stream) {
  const int C = (max_row_len + kChunk - 1) / kChunk;
  MbWs w = carve_ws(ws, num_rows, C > hist_lists ? C : hist_lists);
  w.nh = hist_lists;
  dim3 grid(C, num_rows);
  topk_filter_kernel<<<grid, kMbThreads, 0, stream>>>(logits, ld, row_len, k, idx, w);
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
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&topk_row_kernel<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(sizeof(uint32_t) * kStageElems));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    topk_row_kernel<true><<<num_rows, kSmallThreads, sizeof(uint32_t) * max_row_len, stream>>>(
        logits, ld, row_len, k, idx);
  } else {
    topk_row_kernel<false><<<num_rows, kSmallThreads, 0, stream>>>(logits, ld, row_len, k, idx);
  }
  return hipGetLastError();
}

}  // namespace dsa
