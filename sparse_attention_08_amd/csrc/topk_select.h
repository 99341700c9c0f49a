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
constexpr int kSurvLoads = 8192;           // survivors per workgroup loaded with the chunk counts

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
// wsum: NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const uint32_t s = wsum[w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total,
                                                    BlockScratch<NT> &sh) {
  return block_excl_scan<NT>(v, total, sh.wsum);
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

// ------------------------------------------------------------------------------------
// Selection by the last workgroup to finish scoring a row (score producers that cover
// contiguous chunks of the row, one chunk per workgroup)
// ------------------------------------------------------------------------------------
// Each of the C workgroups of row r scored the positions [c*span, (c+1)*span) of the row and
// published, before counting itself in arrive[r]:
//   * its leading-digit histogram, compressed to the nonzero bins (hcnt, hlist);
//   * its candidates: every position of its chunk whose leading digit is >= b_loc(c), the
//     lowest digit whose count of scores at or above it fits `cap` (kBins when even the top
//     bin does not fit), as (order key, position) pairs in position order; meta = (b_loc, n).
// The k largest scores of the row all have a leading digit >= b*, the digit of the k-th
// largest.  A chunk with b_loc(c) <= b* therefore lists every score of it that survives b*;
// the chunk of a list that does not (more than cap of its scores reach b*) is re-read from
// the score row.  Every value that crosses workgroups is stored with agent scope (written
// through the L2, so the release that publishes it has no dirty lines to write back).
struct SelWs {
  uint32_t *arrive;   // [R]          workgroups of the row that are done (0 between calls)
  uint32_t *hcnt;     // [R][C]       nonzero bins of each chunk's histogram
  uint32_t *hlist;    // [R][C][kBins] (digit << 16 | count) of those bins, ascending
  uint2 *meta;        // [R][C]       (b_loc, number of candidates)
  uint2 *cand;        // [R][C][cap]  (order key, position) candidates, ascending positions
  int C, cap;
};

__host__ __device__ inline size_t sel_ws_bytes(int R, int C, int cap) {
  return align256(sizeof(uint32_t) * (size_t)R) + align256(sizeof(uint32_t) * (size_t)R * C) +
         align256(sizeof(uint32_t) * (size_t)R * C * kBins) + align256(sizeof(uint2) * (size_t)R * C) +
         sizeof(uint2) * (size_t)R * C * cap;
}

// The arrival counters come first: a zero-filled workspace is ready for its first call.
__host__ __device__ inline SelWs carve_sel_ws(void *ws, int R, int C, int cap) {
  uint8_t *p = static_cast<uint8_t *>(ws);
  SelWs w;
  w.arrive = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R);
  w.hcnt = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * C);
  w.hlist = reinterpret_cast<uint32_t *>(p);
  p += align256(sizeof(uint32_t) * (size_t)R * C * kBins);
  w.meta = reinterpret_cast<uint2 *>(p);
  p += align256(sizeof(uint2) * (size_t)R * C);
  w.cand = reinterpret_cast<uint2 *>(p);
  w.C = C;
  w.cap = cap;
  return w;
}

// Stores that other workgroups read within the same kernel: agent scope (write-through).
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint2 *p, uint32_t lo, uint32_t hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), (uint64_t)lo | ((uint64_t)hi << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every store of this wave has completed (the workgroup barrier does not wait for them).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// LDS of the per-chunk publication (any NT): NT/64 scan words and two flags.
struct PublishLds {
  uint32_t wsum[16];
  uint32_t bloc;
  uint32_t last;
};

// The per-workgroup part, called by all NT threads once the chunk's scores are in LDS
// (sc[i] = score of position lo + i, for positions [lo, hi)): writes them to the score row
// `row` (agent scope), builds their leading-digit histogram in `hist` (kBins words of LDS),
// publishes the histogram and the candidates (when `publish`), then counts the workgroup in
// arrive[r].  Returns true in every thread of the workgroup that arrived last.
template <int NT>
__device__ bool publish_chunk(const float *sc, uint32_t *hist, PublishLds &pl, const SelWs &ws,
                              int r, int c, int lo, int hi, float *__restrict__ row,
                              bool publish) {
  static_assert(NT / kWave <= 16 && kBins % NT == 0, "publication shape");
  const int t = threadIdx.x;
  const size_t lc = (size_t)r * ws.C + c;
  for (int i = t; i < kBins; i += NT) hist[i] = 0;
  if (t == 0) pl.bloc = kBins;
  __syncthreads();
  // the scores out to the row, and their histogram (4 consecutive positions per thread)
  for (int p0 = lo; p0 < hi; p0 += 4 * NT) {
    const int p = p0 + 4 * t;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (p + i < hi) {
        const float v = sc[p + i - lo];
        st_agent(row + p + i, v);
        if (publish) atomicAdd(&hist[order_key(v) >> (32 - kD0Bits)], 1u);
      }
  }
  if (publish) {
    __syncthreads();
    constexpr int PER = kBins / NT;
    uint32_t cnt[PER], nz = 0, tot = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      cnt[j] = hist[PER * t + j];
      nz += cnt[j] ? 1u : 0u;
      tot += cnt[j];
    }
    // nonzero bins, ascending
    uint32_t nz_tot;
    uint32_t off = block_excl_scan<NT>(nz, nz_tot, pl.wsum);
    uint32_t *dst = ws.hlist + lc * kBins;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (cnt[j]) st_agent(dst + off++, ((uint32_t)(PER * t + j) << 16) | cnt[j]);
    if (t == 0) st_agent(ws.hcnt + lc, nz_tot);
    // b_loc: the lowest digit d with (scores at digits >= d) <= cap
    uint32_t n_tot;
    const uint32_t pre = block_excl_scan<NT>(tot, n_tot, pl.wsum);
    uint32_t s = n_tot - pre - tot;   // scores in the bins above this thread's
    int mine = kBins;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      s += cnt[j];
      if (s > (uint32_t)ws.cap) break;
      mine = PER * t + j;
    }
    if (mine < kBins) atomicMin(&pl.bloc, (uint32_t)mine);
    __syncthreads();
    const uint32_t bloc = pl.bloc;
    // candidates in position order, 4 consecutive positions per thread and pass
    uint2 *cl = ws.cand + lc * ws.cap;
    uint32_t base = 0;
    for (int p0 = lo; p0 < hi; p0 += 4 * NT) {
      const int p = p0 + 4 * t;
      uint32_t key[4], m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        key[i] = p + i < hi ? order_key(sc[p + i - lo]) : 0u;
        if (p + i < hi && (key[i] >> (32 - kD0Bits)) >= bloc) m |= 1u << i;
      }
      uint32_t ptot;
      uint32_t o = base + block_excl_scan<NT>((uint32_t)__popc(m), ptot, pl.wsum);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((m >> i) & 1u) {
          if (o < (uint32_t)ws.cap) st_agent(cl + o, key[i], (uint32_t)(p + i));
          ++o;
        }
      base += ptot;
    }
    if (t == 0) st_agent(ws.meta + lc, bloc, base < (uint32_t)ws.cap ? base : (uint32_t)ws.cap);
  }
  // release the chunk's scores and publications to the row's last workgroup
  wait_stores();
  __syncthreads();
  if (t == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old =
        __hip_atomic_fetch_add(ws.arrive + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pl.last = old == (uint32_t)ws.C - 1 ? 1u : 0u;
  }
  __syncthreads();
  const bool last = pl.last != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// LDS of the row selection.
template <int NT>
struct SelectLds {
  BlockScratch<NT> sh;
  uint32_t skey[kSurvivorCap];
  int32_t spos[kSurvivorCap];
  uint32_t coff[kMaxChunks + 1];
  uint32_t lmode[kMaxChunks];   // 1: the chunk's survivors come from its list
  uint32_t bstar, above, total, any_fb;
};

// The row's selection, by the last workgroup of the row (all NT threads, after
// publish_chunk returned true): writes the k_eff positions of row r (n scores in `row`)
// to out[0..k) in ascending order, -1 padded, and leaves arrive[r] at zero.
template <int NT>
__device__ void select_published(const SelWs &ws, int r, int n, int k, int span,
                                 const float *__restrict__ row, int32_t *__restrict__ out,
                                 SelectLds<NT> &L) {
  constexpr int kCandMax = 16;      // candidates per thread held in registers
  const int C = ws.C;
  const int t = threadIdx.x;
  if (t == 0) __hip_atomic_store(ws.arrive + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (n <= k) {
    write_all(out, n, k);
    return;
  }
  int tpl = NT;
  while (tpl > 1 && tpl * C > NT) tpl >>= 1;
  const int l = t / tpl, sub = t % tpl;
  const int E = ws.cap / tpl;       // candidates per thread (<= kCandMax, set on the host)
  const bool has = l < C;
  const size_t lc = (size_t)r * C + l;
  // one round of loads: histogram heads, list descriptors and every candidate
  uint32_t hc = 0, he[kListHead];
  uint2 md = make_uint2(0u, 0u);
  uint2 ce[kCandMax];
  const uint32_t *hl = ws.hlist + lc * kBins;
  if (has) {
    hc = ws.hcnt[lc];
    md = ws.meta[lc];
#pragma unroll
    for (int j = 0; j < kListHead; ++j) {
      const int e = sub + tpl * j;
      he[j] = e < kBins ? hl[e] : 0u;
    }
    const uint2 *cl = ws.cand + lc * ws.cap + (size_t)sub * E;
#pragma unroll
    for (int j = 0; j < kCandMax; ++j) ce[j] = j < E ? cl[j] : make_uint2(0u, 0u);
  }
  for (int i = t; i < kBins; i += NT) L.sh.hist[i] = 0;
  __syncthreads();
  if (has) {
#pragma unroll
    for (int j = 0; j < kListHead; ++j)
      if ((uint32_t)(sub + tpl * j) < hc) atomicAdd(&L.sh.hist[he[j] >> 16], he[j] & 0xFFFFu);
    for (uint32_t e = tpl * kListHead + sub; e < hc; e += tpl) {
      const uint32_t v = hl[e];
      atomicAdd(&L.sh.hist[v >> 16], v & 0xFFFFu);
    }
  }
  __syncthreads();
  // b*, the scores above it, and the survivors (digit >= b*)
  {
    constexpr int PER = kBins / NT;
    uint32_t cc[PER], tot = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      cc[j] = L.sh.hist[kBins - 1 - PER * t - j];
      tot += cc[j];
    }
    uint32_t all;
    const uint32_t before = block_excl_scan<NT>(tot, all, L.sh);
    if (before < (uint32_t)k && before + tot >= (uint32_t)k) {
      uint32_t run = before;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (run + cc[j] >= (uint32_t)k) {
          L.bstar = kBins - 1 - PER * t - j;
          L.above = run;
          L.total = run + cc[j];
          break;
        }
        run += cc[j];
      }
    }
    if (t == 0) L.any_fb = 0;
  }
  __syncthreads();
  const uint32_t bstar = L.bstar, above = L.above, M = L.total;
  if (M > (uint32_t)kSurvivorCap) {
    // degenerate score distributions (huge ties around the threshold): the whole row
    select_block<NT>(RowAcc{row}, n, k, out, L.sh, (int)bstar, k - (int)above);
    return;
  }
  if (has && sub == 0) {
    const bool listed = md.x <= bstar;
    L.lmode[l] = listed ? 1u : 0u;
    if (!listed) L.any_fb = 1u;
  }
  __syncthreads();
  if (L.any_fb == 0) {
    // every chunk's survivors are in its list: gather them in position order
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kCandMax; ++j)
      cnt += (j < E && (uint32_t)(sub * E + j) < md.y && (ce[j].x >> (32 - kD0Bits)) >= bstar) ? 1u : 0u;
    uint32_t got;
    uint32_t off = block_excl_scan<NT>(cnt, got, L.sh);
#pragma unroll
    for (int j = 0; j < kCandMax; ++j)
      if (j < E && (uint32_t)(sub * E + j) < md.y && (ce[j].x >> (32 - kD0Bits)) >= bstar &&
          off < (uint32_t)kSurvivorCap) {
        L.skey[off] = ce[j].x;
        L.spos[off] = (int32_t)ce[j].y;
        ++off;
      }
  } else {
    // items: a listed chunk's candidates, else the chunk's positions re-read from the row
    uint32_t ni = 0;
    if (has && sub == 0) {
      const int clen = max(0, min(n, (l + 1) * span) - l * span);
      ni = L.lmode[l] ? md.y : (uint32_t)clen;
    }
    uint32_t T;
    const uint32_t b4 = block_excl_scan<NT>(ni, T, L.sh);
    if (has && sub == 0) L.coff[l] = b4;
    if (t == 0) L.coff[C] = T;
    __syncthreads();
    const uint32_t per = (T + NT - 1) / NT;
    const uint32_t i0 = min(T, (uint32_t)t * per), i1 = min(T, i0 + per);
    auto item = [&](uint32_t i, uint32_t &key, int32_t &pos) {
      const int cl = chunk_of(L.coff, C, i);
      const uint32_t e = i - L.coff[cl];
      if (L.lmode[cl]) {
        const uint2 v = ws.cand[((size_t)r * C + cl) * ws.cap + e];
        key = v.x;
        pos = (int32_t)v.y;
      } else {
        pos = cl * span + (int32_t)e;
        key = order_key(row[pos]);
      }
    };
    uint32_t cnt = 0;
    for (uint32_t i = i0; i < i1; ++i) {
      uint32_t key;
      int32_t pos;
      item(i, key, pos);
      cnt += (key >> (32 - kD0Bits)) >= bstar ? 1u : 0u;
    }
    uint32_t got;
    uint32_t off = block_excl_scan<NT>(cnt, got, L.sh);
    for (uint32_t i = i0; i < i1; ++i) {
      uint32_t key;
      int32_t pos;
      item(i, key, pos);
      if ((key >> (32 - kD0Bits)) >= bstar && off < (uint32_t)kSurvivorCap) {
        L.skey[off] = key;
        L.spos[off] = pos;
        ++off;
      }
    }
  }
  __syncthreads();
  select_block<NT>(SurvivorAcc{L.skey, L.spos}, (int)M, k, out, L.sh, (int)bstar, k - (int)above);
}

}  // namespace dsa
