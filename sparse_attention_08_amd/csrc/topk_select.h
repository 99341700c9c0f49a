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
constexpr int kSelCandPerThread = 16;   // candidates a selecting thread holds (cap <= 16 * tpl)

struct SelWs {
  uint32_t *arrive;   // [R]          workgroups of the row that are done (0 between calls)
  uint32_t *hcnt;     // [R][C]       nonzero bins of each chunk's histogram
  uint32_t *hlist;    // [R][C][kBins] (digit << 16 | count) of those bins, ascending
  uint2 *meta;        // [R][C]       (b_loc, number of candidates)
  uint2 *cand;        // [R][C][cap]  (order key, position) candidates, ascending positions
  int C, cap;         // chunks per row; list capacity (a power of two)
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
// Loads of what other workgroups of the same kernel published: agent scope, so they read
// the coherent copy and the reader needs no cache invalidation (an acquire fence) once it
// has seen the arrival count that follows the publication.
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 ld_agent(const uint2 *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<uint2 *>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
// Every store of this wave has completed (the workgroup barrier does not wait for them).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// LDS of the per-chunk publication (any NT): NT/64 scan words and two flags.
struct PublishLds {
  uint32_t wsum[16];
  uint32_t bloc;
  uint32_t last;
};

// Agent-scope store of 4 consecutive floats at row[p .. p+4) (16-byte aligned), through a
// buffer descriptor of the row's valid scores (stores past them are dropped).
__device__ __forceinline__ void st_agent_x4(const __amdgpu_buffer_rsrc_t &rs, int p, float a, float b,
                                            float c, float d) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, (f32x4v{a, b, c, d})), rs, 4 * p, 0,
                                         16 /* sc1 */);
}

// The per-workgroup part, called by all NT threads once the chunk's scores are in LDS
// (sc[i] = score of position lo + i, for positions [lo, hi)): writes them to the score row
// `row` (agent scope; row[0..len) valid), builds their leading-digit histogram in `hist`
// (kBins words of LDS), publishes the histogram and the candidates (when `publish`), then
// counts the workgroup in arrive[r].  Returns true in every thread of the workgroup that
// arrived last; that workgroup reads the publications with agent-scope loads (ld_agent) or
// after an agent-scope acquire fence.
template <int NT>
__device__ bool publish_chunk(const float *sc, uint32_t *hist, PublishLds &pl, const SelWs &ws,
                              int r, int c, int lo, int hi, int len, float *__restrict__ row,
                              bool publish) {
  static_assert(NT / kWave <= 16 && kBins % NT == 0, "publication shape");
  const int t = threadIdx.x;
  const size_t lc = (size_t)r * ws.C + c;
  if (publish) {
    for (int i = t; i < kBins; i += NT) hist[i] = 0;
    if (t == 0) pl.bloc = kBins;
    __syncthreads();
  }
  // the scores out to the row, and their histogram: 4 consecutive positions per thread
  const bool x4 = ((reinterpret_cast<uintptr_t>(row + lo) & 15) == 0);   // uniform
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(row, (short)0, 4 * len, 0x00020000);
  for (int p0 = lo; p0 < hi; p0 += 4 * NT) {
    const int p = p0 + 4 * t;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p + i < hi ? sc[p + i - lo] : 0.f;
    if (x4) {
      if (p < hi) st_agent_x4(rs, p, v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p + i < hi) st_agent(row + p + i, v[i]);
    }
    if (publish)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p + i < hi) atomicAdd(&hist[order_key(v[i]) >> (32 - kD0Bits)], 1u);
  }
  if (publish) {
    __syncthreads();
    constexpr int PER = kBins / NT;
    static_assert(PER % 4 == 0, "whole 16-byte reads of a thread's bins");
    uint32_t cnt[PER], nz = 0, tot = 0;
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4 *>(hist + PER * t + j);
      cnt[j] = v.x;
      cnt[j + 1] = v.y;
      cnt[j + 2] = v.z;
      cnt[j + 3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      nz += cnt[j] ? 1u : 0u;
      tot += cnt[j];
    }
    // one scan for both the nonzero-bin offsets (high half) and the score counts (low half;
    // a chunk holds fewer than 65536 scores)
    uint32_t both;
    const uint32_t pre = block_excl_scan<NT>((nz << 16) | tot, both, pl.wsum);
    uint32_t off = pre >> 16;
    uint32_t *dst = ws.hlist + lc * kBins;
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (cnt[j]) st_agent(dst + off++, ((uint32_t)(PER * t + j) << 16) | cnt[j]);
    if (t == 0) st_agent(ws.hcnt + lc, both >> 16);
    // b_loc: the lowest digit d with (scores at digits >= d) <= cap
    uint32_t s = (both & 0xFFFFu) - (pre & 0xFFFFu) - tot;   // scores in the bins above
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
  return pl.last != 0;
}

// LDS of the row selection.
template <int NT>
struct SelectLds {
  uint32_t hist[kBins];               // merged leading-digit histogram
  uint32_t hist1[1 << kD1Bits];       // second digit of the boundary bin's survivors
  uint32_t hist2[1 << kD2Bits];       // third digit of the boundary's second-digit bin
  uint32_t wsum[NT / kWave];
  uint32_t wcnt[2][NT / kWave];
  uint32_t skey[kSurvivorCap];
  int32_t spos[kSurvivorCap];
  uint32_t coff[kMaxChunks + 1];
  uint32_t lmode[kMaxChunks];         // 1: the chunk's survivors come from its list
  uint32_t bstar, above, total, any_fb, d1, need1, T, need_eq;
};

// The digit of the `need`-th largest among the counts h[0..NB) taken from the top, and how
// many lie strictly above it; one wave.  Lane l first sums the NB/64 bins of its range
// (descending ranges: lane 0 holds the top), reading them in a lane-rotated order so the
// wave's reads hit distinct LDS banks; the wave then scans the lane totals, and the 64 lanes
// read the range that holds the answer, one bin each, and scan it.
template <int NB>
__device__ __forceinline__ void wave_find_digit(const uint32_t *h, uint32_t need, uint32_t &digit,
                                                uint32_t &above) {
  constexpr int PER = NB / kWave;
  static_assert(PER <= kWave, "one bin per lane in the final step");
  const int lane = threadIdx.x & 63;
  const int top = NB - 1 - PER * lane;   // this lane's range: bins top, top-1, ..., top-PER+1
  uint32_t tot = 0;
#pragma unroll 8
  for (int j = 0; j < PER; ++j) tot += h[top - ((j + lane) & (PER - 1))];
  const uint32_t inc = wave_incl_scan(tot);
  const uint64_t hit = __ballot(inc >= need);
  const int L = hit ? __ffsll((long long)hit) - 1 : kWave - 1;   // the range holding it
  const uint32_t before = (uint32_t)__shfl((int)(inc - tot), L, kWave);
  // bins of range L, descending: lane j takes bin top(L) - j
  const int tl = NB - 1 - PER * L;
  const uint32_t c = lane < PER ? h[tl - lane] : 0u;
  const uint32_t cinc = before + wave_incl_scan(c);
  const uint64_t hit2 = __ballot(lane < PER && cinc >= need);
  const int j = hit2 ? __ffsll((long long)hit2) - 1 : PER - 1;
  digit = (uint32_t)(tl - j);
  above = (uint32_t)__shfl((int)(cinc - c), j, kWave);
}

// Rare paths of the row selection, kept out of line (the selection runs once per row, from
// cold instruction caches, so its common path is kept short).
// Degenerate score distributions (more survivors than the LDS holds): the whole row.
template <int NT>
__device__ __attribute__((noinline)) void select_whole_row(const float *row, int n, int k,
                                                           int32_t *out, BlockScratch<NT> *sh,
                                                           int bstar, int need) {
  // the row's scores come from other workgroups of the kernel: plain loads after an acquire
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  select_block<NT>(RowAcc{row}, n, k, out, *sh, bstar, need);
}
// Some chunk's list misses survivors: the survivors of every chunk, from its list or re-read
// from its scores, into skey/spos in position order.  coff and lmode: per-chunk LDS arrays
// (lmode[c] = 1 when chunk c's list holds its survivors); ni: this thread's chunk item count
// (threads lead of chunk l), wsum: NT/64 LDS words.  The items (a listed chunk's candidates,
// another chunk's positions) are taken in position order, each thread a run of consecutive
// items whose loads are all issued before any is used; one scan per run of kRun items a thread.
template <int NT>
__device__ __attribute__((noinline)) void gather_rereads(const SelWs ws, int r, int n, int span,
                                                         const float *row, uint32_t bstar,
                                                         uint32_t ni, bool lead, int l,
                                                         uint32_t *coff, const uint32_t *lmode,
                                                         uint32_t *wsum, uint32_t *skey,
                                                         int32_t *spos) {
  constexpr int kRun = 16;
  // lists and scores come from other workgroups of the kernel: plain loads after an acquire
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int C = ws.C;
  const int t = threadIdx.x;
  uint32_t T;
  const uint32_t b4 = block_excl_scan<NT>(ni, T, wsum);
  if (lead) coff[l] = b4;
  if (t == 0) coff[C] = T;
  __syncthreads();
  uint32_t base = 0;
  for (uint32_t p0 = 0; p0 < T; p0 += (uint32_t)NT * kRun) {
    const uint32_t i0 = p0 + (uint32_t)t * kRun;
    uint32_t key[kRun];
    int32_t pos[kRun];
    uint32_t from_row = 0;   // items read from the score row (converted once loaded)
    int cl = i0 < T ? chunk_of(coff, C, i0) : 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const uint32_t i = i0 + j;
      while (cl + 1 < C && coff[cl + 1] <= i) ++cl;
      const uint32_t e = i - coff[cl];
      if (i >= T) {
        key[j] = 0u;
        pos[j] = -1;
      } else if (lmode[cl]) {
        const uint2 v = ws.cand[((size_t)r * C + cl) * ws.cap + e];
        key[j] = v.x;
        pos[j] = (int32_t)v.y;
      } else {
        pos[j] = cl * span + (int32_t)e;
        key[j] = __float_as_uint(row[pos[j]]);
        from_row |= 1u << j;
      }
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      if ((from_row >> j) & 1u) key[j] = order_key(__uint_as_float(key[j]));
      cnt += (pos[j] >= 0 && (key[j] >> (32 - kD0Bits)) >= bstar) ? 1u : 0u;
    }
    uint32_t got;
    uint32_t off = base + block_excl_scan<NT>(cnt, got, wsum);
#pragma unroll
    for (int j = 0; j < kRun; ++j)
      if (pos[j] >= 0 && (key[j] >> (32 - kD0Bits)) >= bstar) {
        if (off < (uint32_t)kSurvivorCap) {
          skey[off] = key[j];
          spos[off] = pos[j];
        }
        ++off;
      }
    base += got;
  }
}

// The row's selection (all NT threads), once every chunk of row r is published: writes the
// k_eff positions of the row (n scores in `row`) to out[0..k) in ascending order, -1 padded.
// out may be global or LDS (not inside L).
template <int NT>
__device__ void select_published(const SelWs &ws, int r, int n, int k, int span,
                                 const float *__restrict__ row, int32_t *out, SelectLds<NT> &L) {
  constexpr int kCandMax = kSelCandPerThread;   // candidates per lane held in registers
  constexpr int NW = NT / kWave;
  const int C = ws.C;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  if (n <= k) {
    write_all(out, n, k);
    return;
  }
  int tpl = NT;
  while (tpl > 1 && tpl * C > NT) tpl >>= 1;
  const int l = t / tpl, sub = t % tpl;
  const bool has = l < C;
  const size_t lc = (size_t)r * C + l;
  // one round of loads: histogram heads (tpl threads per list), list descriptors (thread c
  // for list c) and every candidate slot of the row's lists, read wave-contiguously: wave w
  // takes the J * 64 slots from w * J * 64, lane i every 64th of them (C * cap <= 16 NT)
  const int J = (C * ws.cap + NT - 1) / NT;
  uint32_t hc = 0, he[kListHead];
  const uint32_t *hl = ws.hlist + lc * kBins;
  if (has) {
    hc = ld_agent(ws.hcnt + lc);
#pragma unroll
    for (int j = 0; j < kListHead; ++j) {
      const int e = sub + tpl * j;
      he[j] = e < kBins ? ld_agent(hl + e) : 0u;
    }
  }
  const uint2 md = t < C ? ld_agent(ws.meta + (size_t)r * C + t) : make_uint2(0u, 0u);
  const uint2 *crow = ws.cand + (size_t)r * C * ws.cap;
  const int e0 = wave * J * kWave + lane;
  uint2 ce[kCandMax];
#pragma unroll
  for (int j = 0; j < kCandMax; ++j) {
    const int e = e0 + kWave * j;
    ce[j] = (j < J && e < C * ws.cap) ? ld_agent(crow + e) : make_uint2(0u, 0u);
  }
  for (int i = t; i < kBins; i += NT) L.hist[i] = 0;
  for (int i = t; i < (1 << kD1Bits); i += NT) L.hist1[i] = 0;
  for (int i = t; i < (1 << kD2Bits); i += NT) L.hist2[i] = 0;
  if (t == 0) L.any_fb = 0;
  if (t < C) L.coff[t] = md.y;   // candidates of list t (coff is reused by the re-read path)
  __syncthreads();
  if (has) {
#pragma unroll
    for (int j = 0; j < kListHead; ++j)
      if ((uint32_t)(sub + tpl * j) < hc) atomicAdd(&L.hist[he[j] >> 16], he[j] & 0xFFFFu);
    for (uint32_t e = tpl * kListHead + sub; e < hc; e += tpl) {
      const uint32_t v = ld_agent(hl + e);
      atomicAdd(&L.hist[v >> 16], v & 0xFFFFu);
    }
  }
  __syncthreads();
  // b*, the scores above it, and the survivors (digit >= b*): one wave
  if (wave == 0) {
    uint32_t d, ab;
    wave_find_digit<kBins>(L.hist, (uint32_t)k, d, ab);
    if (lane == 0) {
      L.bstar = d;
      L.above = ab;
      L.total = ab + L.hist[d];
    }
  }
  __syncthreads();
  const uint32_t bstar = L.bstar, above = L.above, M = L.total;
  if (__builtin_expect(M > (uint32_t)kSurvivorCap, 0)) {
    // degenerate score distributions (huge ties around the threshold): the whole row
    select_whole_row<NT>(row, n, k, out, reinterpret_cast<BlockScratch<NT> *>(L.skey), (int)bstar,
                         k - (int)above);
    return;
  }
  if (t < C) {
    const bool listed = md.x <= bstar;
    L.lmode[t] = listed ? 1u : 0u;
    if (!listed) L.any_fb = 1u;
  }
  __syncthreads();
  if (__builtin_expect(L.any_fb == 0, 1)) {
    // every chunk's survivors are in its list: keep the valid slots that reach b*, in slot
    // order (a wave's span, then the waves in turn).  Slot e is entry e % cap of list
    // e / cap (cap is a power of two); the list counts are read from LDS in one batch.
    const int csh = 31 - __builtin_clz((uint32_t)ws.cap);
    const int n_slot = C << csh;
    uint32_t cnt[kCandMax];
#pragma unroll
    for (int j = 0; j < kCandMax; ++j) {
      const int e = e0 + kWave * j;
      cnt[j] = (j < J && e < n_slot) ? L.coff[e >> csh] : 0u;
    }
    uint32_t keepm = 0, wc = 0;
#pragma unroll
    for (int j = 0; j < kCandMax; ++j) {
      const int e = e0 + kWave * j;
      const bool keep = (uint32_t)(e & (ws.cap - 1)) < cnt[j] && (ce[j].x >> (32 - kD0Bits)) >= bstar;
      keepm |= keep ? 1u << j : 0u;
      wc += __popcll(__ballot(keep));
    }
    if (lane == 0) L.wcnt[0][wave] = wc;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += L.wcnt[0][w];
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < kCandMax; ++j) {
      const bool keep = (keepm >> j) & 1u;
      const uint64_t m = __ballot(keep);
      const uint32_t o = off + __popcll(m & lt);
      if (keep && o < (uint32_t)kSurvivorCap) {
        L.skey[o] = ce[j].x;
        L.spos[o] = (int32_t)ce[j].y;
      }
      off += __popcll(m);
    }
  } else {
    uint32_t ni = 0;
    if (has && sub == 0) {
      const int clen = max(0, min(n, (l + 1) * span) - l * span);
      ni = L.lmode[l] ? L.coff[l] : (uint32_t)clen;
    }
    __syncthreads();   // the list counts in coff are read before it holds the item offsets
    gather_rereads<NT>(ws, r, n, span, row, bstar, ni, has && sub == 0, l, L.coff, L.lmode, L.wsum,
                       L.skey, L.spos);
  }
  __syncthreads();
  // the key T of the k-th largest: its second and third digits among the boundary bin's
  // survivors (need1 of them belong to the result)
  const uint32_t need1 = (uint32_t)k - above;
  for (int i0 = t; i0 < (int)M; i0 += 4 * NT) {
    uint32_t u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = i0 + q * NT < (int)M ? L.skey[i0 + q * NT] : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + q * NT < (int)M && (u[q] >> (32 - kD0Bits)) == bstar)
        atomicAdd(&L.hist1[(u[q] >> kD2Bits) & ((1u << kD1Bits) - 1)], 1u);
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t d, ab;
    wave_find_digit<(1 << kD1Bits)>(L.hist1, need1, d, ab);
    if (lane == 0) {
      L.d1 = d;
      L.need1 = need1 - ab;
    }
  }
  __syncthreads();
  const uint32_t pre2 = (bstar << kD1Bits) | L.d1, need2 = L.need1;
  for (int i0 = t; i0 < (int)M; i0 += 4 * NT) {
    uint32_t u[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = i0 + q * NT < (int)M ? L.skey[i0 + q * NT] : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + q * NT < (int)M && (u[q] >> kD2Bits) == pre2)
        atomicAdd(&L.hist2[u[q] & ((1u << kD2Bits) - 1)], 1u);
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t d, ab;
    wave_find_digit<(1 << kD2Bits)>(L.hist2, need2, d, ab);
    if (lane == 0) {
      L.T = (pre2 << kD2Bits) | d;
      L.need_eq = need2 - ab;
    }
  }
  __syncthreads();
  // ordered write: wave w owns a contiguous span of the survivors
  const uint32_t T = L.T;
  const int32_t need_eq = (int32_t)L.need_eq;
  const int wspan = ((((int)M + NW - 1) / NW) + 63) & ~63;
  const int wlo = wave * wspan, whi = min((int)M, wlo + wspan);
  // (4 survivors a lane per round, their LDS reads issued together)
  constexpr int kU = 4;
  uint32_t gt_cnt = 0, eq_cnt = 0;
  for (int b0 = wlo; b0 < whi; b0 += kU * kWave) {
    uint32_t u[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int i = b0 + q * kWave + lane;
      u[q] = i < whi ? L.skey[i] : 0u;
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const bool in = b0 + q * kWave + lane < whi;
      gt_cnt += __popcll(__ballot(in && u[q] > T));
      eq_cnt += __popcll(__ballot(in && u[q] == T));
    }
  }
  if (lane == 0) {
    L.wcnt[0][wave] = gt_cnt;
    L.wcnt[1][wave] = eq_cnt;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const int32_t take = max(0, min((int32_t)L.wcnt[1][w], need_eq - (int32_t)eq_before));
    sel_before += L.wcnt[0][w] + (uint32_t)take;
    eq_before += L.wcnt[1][w];
  }
  const uint64_t lt = lanemask_lt();
  for (int b0 = wlo; b0 < whi; b0 += kU * kWave) {
    uint32_t u[kU];
    int32_t ps[kU];
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int i = b0 + q * kWave + lane;
      u[q] = i < whi ? L.skey[i] : 0u;
      ps[q] = i < whi ? L.spos[i] : 0;
    }
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const bool in = b0 + q * kWave + lane < whi;
      const bool gt = in && u[q] > T;
      const bool eq = in && u[q] == T;
      const uint64_t eq_mask = __ballot(eq);
      const uint32_t eq_rank = eq_before + __popcll(eq_mask & lt);
      const bool sel = gt || (eq && eq_rank < (uint32_t)need_eq);
      const uint64_t sel_mask = __ballot(sel);
      if (sel) out[sel_before + __popcll(sel_mask & lt)] = ps[q];
      eq_before += __popcll(eq_mask);
      sel_before += __popcll(sel_mask);
    }
  }
}

}  // namespace dsa
