// topk_select.h -- the exact radix selection shared by the top-k kernels and by the
// attention kernel that finishes the selection of its own row ("DeepSeek-V3.2 技术报告
// 摘要", section 1, DSA ② Fine-grained Token Selection).
//
// Keys are order-preserving 32-bit images of the scores (-0 folded onto +0); a radix select
// with digits of 12, 10 and 10 bits finds the key T of the k-th largest score and how many
// keys equal to T are still needed; an ordered pass writes every position with key > T
// plus the lowest-positioned keys == T, in ascending position order.
#pragma once
#include "dsa_device.h"

namespace dsa {

constexpr int kD0Bits = kLeadDigitBits, kD1Bits = 10, kD2Bits = 10;
constexpr int kBins = 1 << kD0Bits;        // 4096
constexpr int kChunk = 4096;               // scores per workgroup in the few-row schedule
constexpr int kSurvivorCap = 10240;        // survivors selected in LDS (80 KB)
constexpr int kMaxChunks = 256;            // chunked schedule handles rows up to 1M scores
constexpr int kListHead = 8;               // histogram entries per thread loaded with the counts
#ifndef DSA_SURV_LOADS
#define DSA_SURV_LOADS 8192
#endif
constexpr int kSurvLoads = DSA_SURV_LOADS;  // survivors per workgroup loaded with the chunk counts

// ------------------------------------------------------------------------------------
// block-wide helpers
// ------------------------------------------------------------------------------------
// P16: two 16-bit bin counts per word (every count stays below 65536, i.e. fewer than
// 65536 keys), which halves the histogram's LDS.
template <int NT, bool P16 = false>
struct BlockScratch {
  uint32_t hist[P16 ? kBins / 2 : kBins];
  uint32_t wsum[NT / kWave];
  uint32_t wcnt[2][NT / kWave];
  uint32_t prefix, mask;
  int32_t need;
  uint32_t flag;
};

// Exclusive prefix sum over the block's threads of v; returns it and the block total.
template <int NT, bool P16>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total,
                                                    BlockScratch<NT, P16> &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
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

// The digit holding the need-th largest key among those matching (key & mask) == prefix,
// from a histogram of the digit (key >> shift) & (2^BITS - 1) already counted in sh.hist;
// updates prefix, mask and need.
template <int NT, int BITS, bool P16>
__device__ void radix_resolve(int shift, BlockScratch<NT, P16> &sh) {
  constexpr int NB = 1 << BITS;
  constexpr int PER = NB / NT;             // consecutive bins owned per thread
  static_assert(NB % NT == 0, "bins must split evenly");
  const uint32_t prefix = sh.prefix, mask = sh.mask;
  // thread t owns bins NB-1-PER*t-j (j < PER): descending digit order across threads
  uint32_t c[PER], tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = NB - 1 - PER * threadIdx.x - j;
    if constexpr (P16) c[j] = (sh.hist[b >> 1] >> (16 * (b & 1))) & 0xFFFFu;
    else c[j] = sh.hist[b];
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

// One radix digit: histogram of digit (key >> shift) & (2^BITS - 1) over the keys that
// match (key & mask) == prefix, then the digit holding the need-th largest key.
template <int NT, int BITS, bool P16, class Acc>
__device__ void radix_digit(const Acc &acc, int n, int shift, BlockScratch<NT, P16> &sh) {
  constexpr int NB = 1 << BITS;
  constexpr int NW = P16 ? NB / 2 : NB;    // histogram words
  for (int i = threadIdx.x; i < NW; i += NT) sh.hist[i] = 0;
  __syncthreads();
  const uint32_t prefix = sh.prefix, mask = sh.mask;
  // four keys a thread per round, their reads issued together
  for (int i0 = threadIdx.x; i0 < n; i0 += 4 * NT) {
    uint32_t u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = i0 + q * NT < n ? acc.key(i0 + q * NT) : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + q * NT < n && (u[q] & mask) == prefix) {
        const uint32_t d = (u[q] >> shift) & (NB - 1);
        if constexpr (P16) atomicAdd(&sh.hist[d >> 1], 1u << (16 * (d & 1)));
        else atomicAdd(&sh.hist[d], 1u);
      }
  }
  __syncthreads();
  radix_resolve<NT, BITS>(shift, sh);
}

// The rest of select_block once sh holds the prefix, mask and need after the first digit.
template <int NT, bool P16, class Acc>
__device__ void select_after_first_digit(const Acc &acc, int n, int32_t *__restrict__ out,
                                         BlockScratch<NT, P16> &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  radix_digit<NT, kD1Bits>(acc, n, kD2Bits, sh);
  radix_digit<NT, kD2Bits>(acc, n, 0, sh);
  const uint32_t T = sh.prefix;
  const int32_t need_eq = sh.need;
  // ordered write: wave w owns a contiguous span; counts, wave offsets, then ballots (four
  // keys a lane per round, their reads issued together)
  constexpr int NW = NT / kWave;
  constexpr int kU = 4;
  const int span = (((n + NW - 1) / NW) + 63) & ~63;
  const int lo = wave * span, hi = min(n, lo + span);
  uint32_t gt_cnt = 0, eq_cnt = 0;
  for (int base = lo; base < hi; base += kU * kWave) {
    uint32_t u[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int i = base + q * kWave + lane;
      u[q] = i < hi ? acc.key(i) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const bool in = base + q * kWave + lane < hi;
      gt_cnt += __popcll(__ballot(in && u[q] > T));
      eq_cnt += __popcll(__ballot(in && u[q] == T));
    }
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
  for (int base = lo; base < hi; base += kU * kWave) {
    uint32_t u[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int i = base + q * kWave + lane;
      u[q] = i < hi ? acc.key(i) : 0u;
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int i = base + q * kWave + lane;
      const bool gt = i < hi && u[q] > T;
      const bool eq = i < hi && u[q] == T;
      const uint64_t eq_mask = __ballot(eq);
      const uint32_t eq_rank = eq_before + __popcll(eq_mask & lt);
      const bool sel = gt || (eq && eq_rank < (uint32_t)need_eq);
      const uint64_t sel_mask = __ballot(sel);
      if (sel) out[sel_before + __popcll(sel_mask & lt)] = acc.pos(i);
      eq_before += __popcll(eq_mask);
      sel_before += __popcll(sel_mask);
    }
  }
}

// Exact top-k of n keys given by acc (key(i), pos(i); items in ascending position
// order), written to out[0..k) in ascending position order.  Requires n > k, and
// n < 65536 with a 16-bit histogram (P16).
// When first_digit >= 0 the caller already knows the 12-bit digit of T and that
// `need_in_digit` keys with that digit belong to the result.
template <int NT, bool P16, class Acc>
__device__ void select_block(const Acc &acc, int n, int k, int32_t *__restrict__ out,
                             BlockScratch<NT, P16> &sh, int first_digit = -1,
                             int need_in_digit = 0) {
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
  select_after_first_digit<NT>(acc, n, out, sh);
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

// ------------------------------------------------------------------------------------
// the last step of the few-row schedule, for any workgroup size NT >= kMaxChunks
// ------------------------------------------------------------------------------------
// The loads of a row's last step, issued together: b* and the number of scores above it,
// and each chunk's survivor count with its first survivors (tpc threads per chunk).
template <int NT>
struct SurvivorLoads {
  static constexpr int kHead = kSurvLoads / NT;   // per thread
  int bstar, above, tpc, ch, sub;
  uint32_t cnt;
  uint2 head[kHead];
};

// The few-row schedule's arrays in a fused workspace whose histogram lists came from the
// score producer (hist_lists per row).
inline MbWs topk_chunk_ws(void *ws, int num_rows, int max_row_len, int hist_lists) {
  const int C = (max_row_len + kChunk - 1) / kChunk;
  MbWs w = carve_ws(ws, num_rows, C > hist_lists ? C : hist_lists);
  w.nh = hist_lists;
  return w;
}

// nblk: chunks to cover, at least those of the row (extra chunks are read, not used).
template <int NT>
__device__ __forceinline__ SurvivorLoads<NT> issue_survivor_loads(const MbWs &ws, int r, int nblk) {
  static_assert(NT >= kMaxChunks, "a thread per chunk at least");
  SurvivorLoads<NT> L;
  L.bstar = (int)ws.meta[2 * r];
  L.above = (int)ws.meta[2 * r + 1];
  int tpc = NT;
  while (tpc > 1 && tpc * nblk > NT) tpc >>= 1;
  L.tpc = tpc;
  L.ch = threadIdx.x / tpc;
  L.sub = threadIdx.x % tpc;
  L.cnt = 0;
  if (L.ch < nblk) {
    const uint2 *cl = ws.slist + ((size_t)r * ws.C + L.ch) * kChunk;
    L.cnt = ws.scnt[(size_t)r * ws.C + L.ch];
#pragma unroll
    for (int j = 0; j < L.kHead; ++j) {
      const int e = L.sub + tpc * j;
      L.head[j] = e < kChunk ? cl[e] : make_uint2(0u, 0u);   // within the chunk's list
    }
  }
  return L;
}

// Exact top-k of row r (n > k scores) from its survivors: gathered into LDS (skey, spos:
// kSurvivorCap each; coff: kMaxChunks + 1), the last two digits, and the ordered write of
// the k positions to out (global or LDS).  Rows whose survivors exceed the LDS arrays fall
// back to a select over the whole score row.
template <int NT>
__device__ void select_from_survivors(const SurvivorLoads<NT> &L, const float *__restrict__ logits,
                                      int64_t ld, const MbWs &ws, int r, int n, int k,
                                      int32_t *out, BlockScratch<NT> &sh, uint32_t *skey,
                                      int32_t *spos, uint32_t *coff) {
  const int nblk = (n + kChunk - 1) / kChunk;
  {
    uint32_t total;
    const uint32_t before = block_excl_scan<NT>((L.sub == 0 && L.ch < nblk) ? L.cnt : 0u, total, sh);
    if (L.sub == 0 && L.ch < nblk) coff[L.ch] = before;
    if (threadIdx.x == 0) coff[nblk] = total;
  }
  __syncthreads();
  const int M = (int)coff[nblk];
  if (M <= kSurvivorCap) {
    if (L.ch < nblk) {
      const int dst = (int)coff[L.ch];
#pragma unroll
      for (int j = 0; j < L.kHead; ++j) {
        const uint32_t e = L.sub + L.tpc * j;
        if (e < L.cnt) {
          skey[dst + e] = L.head[j].x;
          spos[dst + e] = (int32_t)L.head[j].y;
        }
      }
      const uint2 *cl = ws.slist + ((size_t)r * ws.C + L.ch) * kChunk;
      for (uint32_t e = L.tpc * L.kHead + L.sub; e < L.cnt; e += L.tpc) {
        const uint2 v = cl[e];
        skey[dst + e] = v.x;
        spos[dst + e] = (int32_t)v.y;
      }
    }
    __syncthreads();
    select_block<NT>(SurvivorAcc{skey, spos}, M, k, out, sh, L.bstar, k - L.above);
  } else {
    // degenerate score distributions (huge ties around the threshold): whole row
    select_block<NT>(RowAcc{logits + (int64_t)r * ld}, n, k, out, sh, L.bstar, k - L.above);
  }
}

}  // namespace dsa
