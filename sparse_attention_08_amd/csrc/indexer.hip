// indexer.hip -- lightning-indexer scores on gfx950.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:]) over the preceding tokens s of the
// query's sequence ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ① Lightning Indexer:
// a few indexer heads, one key per token shared by all heads, FP8 supported).
//
// Decode-shaped work (few query rows, long contexts) is bound by the key stream from
// HBM: every key byte is read once and meets 64 heads (64 flop/B in bf16, 128 flop/B
// in fp8), far under the MFMA ridge.  The MFMA kernel therefore deals each row's keys to
// many waves in 4 KB groups, keeps the row's 64x128 query block resident in registers as
// MFMA operands, streams the groups through a small private LDS ring per wave with
// global->LDS loads (the next groups are in flight while one is multiplied), and fuses
// ReLU, the head weights, the fp8 scales and the 64-head sum into the MFMA epilogue.
// The same kernel serves every batch shape of fp8 keys and the bf16 batches with few rows
// per sequence (decode, multi-token decode); indexer_prefill.hip shares key tiles between
// rows for bf16 prefill.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path (any small H, D): one thread per key, plain fp32 FMA.  This is the
// exactness path (checked at 1e-5 relative) and is not tuned.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void indexer_f32_kernel(RowsDev rows, int R, int H, int D,
                                                          const float *__restrict__ q,
                                                          const float *__restrict__ k,
                                                          const float *__restrict__ w,
                                                          float *__restrict__ logits, int64_t ld) {
  extern __shared__ float smem[];   // q row [H*D] then w row [H]
  const int r = grid_row();
  if (r >= R) return;
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
  const dim3 grid = row_grid((rh.max_row_len + 255) / 256, rh.num_rows);
  size_t shm = sizeof(float) * ((size_t)H * D + H);
  // the query block and weights of the largest supported shape (64 heads x 256 dims: 65,792
  // bytes) exceed the default 64 KB of dynamic LDS
  constexpr int kMaxShm = (int)sizeof(float) * (64 * 256 + 64);
  static std::atomic<uint64_t> lds_set[2];
  hipError_t e = paged ? ensure_dynamic_lds(&indexer_f32_kernel<true>, kMaxShm, lds_set[1])
                       : ensure_dynamic_lds(&indexer_f32_kernel<false>, kMaxShm, lds_set[0]);
  if (e != hipSuccess) return e;
  if (paged)
    indexer_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, rh.num_rows, H, D, q, k, w, logits, ld);
  else
    indexer_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, rh.num_rows, H, D, q, k, w, logits, ld);
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
// Epilogue per tile: ReLU and the head weights w' (w' = w * q_scale for fp8) summed over
// the 64 heads by two bf16 MFMAs with the weights as the A operand (head_sum); fp8 then
// multiplies by the key's scale.
// ------------------------------------------------------------------------------------
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;



// A group is 8 KB of keys: 64 fp8 keys or 32 bf16 keys (U = 4 or 2 MFMA tiles of 16).
// Each wave streams its span of keys through a private ring of kDepth LDS slots, filled
// by direct global->LDS loads (global_load_lds_dwordx4: lane l of an instruction lands
// at slot + 1024*j + 16*l), so keys never pass through VGPRs and kDepth-1 groups are in
// flight while one is multiplied.  Each load instruction covers 1 KB of whole cache
// lines.  Inside a slot, key k's 16-byte chunk x is stored at chunk x ^ (k & 7): the
// MFMA operand reads (8 keys at the same logical chunk per LDS cycle) hit 8 distinct
// bank groups.  The swizzle is applied on the global side, by choosing which chunk
// each lane fetches.
#ifndef DSA_IDX_SWZ
#define DSA_IDX_SWZ 1
#endif
// XOR applied to the 16-byte chunk index of key `key` (low 3 bits for 128-byte fp8 rows,
// low 4 bits for 256-byte bf16 rows): 16 consecutive keys read at one logical chunk land
// on 16 distinct 16-byte bank groups.
template <bool FP8>
__device__ __forceinline__ int key_swz(int key) {
  if constexpr (DSA_IDX_SWZ == 0) return key & 7;
  if constexpr (FP8) return ((key >> 1) & 7) ^ ((key & 1) << 2);
  return key & 15;
}
// Launch shape (measured on MI355X): 4 KB key groups; fp8 keys with 16 waves per workgroup
// and 2-slot rings, bf16 keys (more registers per wave) with 8 waves and 3-slot rings; the
// grid is sized for about 256 workgroups.
#ifndef DSA_IDX_WAVES_FP8
#define DSA_IDX_WAVES_FP8 16
#endif
#ifndef DSA_IDX_DEPTH_FP8
#define DSA_IDX_DEPTH_FP8 2
#endif
#ifndef DSA_IDX_WAVES_BF16
#define DSA_IDX_WAVES_BF16 8
#endif
#ifndef DSA_IDX_DEPTH_BF16
#define DSA_IDX_DEPTH_BF16 3
#endif
#ifndef DSA_IDX_BLOCKS
#define DSA_IDX_BLOCKS 256
#endif
#ifndef DSA_IDX_GROUP_BYTES_FP8
#define DSA_IDX_GROUP_BYTES_FP8 4096
#endif
#ifndef DSA_IDX_GROUP_BYTES_BF16
#define DSA_IDX_GROUP_BYTES_BF16 4096
#endif

template <bool FP8>
struct IdxCfg {
  static constexpr int kRowBytes = kIdxDim * (FP8 ? 1 : 2);   // 128 / 256
  static constexpr int kGroupBytes = FP8 ? DSA_IDX_GROUP_BYTES_FP8 : DSA_IDX_GROUP_BYTES_BF16;
  static constexpr int kKeys = kGroupBytes / kRowBytes;        // keys per group (fp8: 32 at 4 KB)
  static constexpr int kTiles = kKeys / 16;                    // 16-key MFMA tiles per group
  static constexpr int kChunks = kRowBytes / 64;               // 16-byte chunks per lane per key
  static constexpr int kSlotBytes = kGroupBytes + (FP8 ? 256 : 0);   // keys (+ 64 scales)
  static constexpr int kWaves = FP8 ? DSA_IDX_WAVES_FP8 : DSA_IDX_WAVES_BF16;   // per workgroup
  static constexpr int kDepth = FP8 ? DSA_IDX_DEPTH_FP8 : DSA_IDX_DEPTH_BF16;   // ring slots per wave
  static_assert(kKeys % 16 == 0 && kKeys >= 16 && kKeys <= 64, "a group is 1 to 4 MFMA tiles");
};

typedef void __attribute__((address_space(3))) *lds_void_ptr;

// s_waitcnt immediate that waits for at most n outstanding vector-memory operations and
// leaves the export and LDS/scalar counters unconstrained (gfx9 field layout).
constexpr int vmcnt_only(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

// Global->LDS loads of 16 (keys) and 4 (fp8 scales) bytes per lane: lane l lands at
// lds + l * size.  When every row has a sequence of its own, each key is read once and the
// key loads carry the non-temporal hint, which keeps the scores and the attention's cache
// lines in L2 and the Infinity Cache for the later stages (measured: plain loads cost 3 to
// 10 us per decode step).  When rows share sequences (several query tokens per sequence)
// the key loads are plain: rows of one sequence read the same keys at about the same time
// from workgroups on the same XCD, and the later reads hit in L2 (measured: two rows per
// sequence then cost about as much as one).
// Written as two-instruction asm statements rather than the builtin: the compiler treats
// every LDS write it cannot disambiguate from a pending global->LDS load as aliasing it
// and would wait for all of them first (draining the rings).  The instructions write no
// register and consume their operands at issue; the kernel waits for the data with
// explicit vmcnt counts (loads complete in order) before reading a slot.
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
}
template <bool NT>
__device__ __forceinline__ void dma16(const void *g, void *lds) {
  if constexpr (NT)
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g),
                     "s"(lds_addr(lds))
                     : "memory");
  else
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                     "s"(lds_addr(lds))
                     : "memory");
}
__device__ __forceinline__ void dma4(const void *g, void *lds) {
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(lds))
                   : "memory");
}

// Per-lane constant part of a group's DMA addresses: for key instruction j, the key of the
// group this lane's 16 bytes belong to and the byte offset of its source chunk.
template <bool FP8>
struct DmaLane {
  static constexpr int kJ = IdxCfg<FP8>::kGroupBytes / 1024;
  int key[kJ];
  int byte[kJ];
  __device__ __forceinline__ void init(int lane) {
    using C = IdxCfg<FP8>;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int pos = 1024 * j + 16 * lane;             // byte position inside the slot
      key[j] = pos / C::kRowBytes;
      const int chunk = (pos % C::kRowBytes) >> 4;      // physical chunk
      byte[j] = key[j] * C::kRowBytes + 16 * (chunk ^ key_swz<FP8>(key[j]));
    }
  }
};

// Issues the loads of the key group starting at position s0 (< row length) into `slot`.
// base_row: contiguous layout, cache row of position 0; paged layout: page holds the cache
// page of the group (a group never crosses a 64-token page).  Keys past s_last (the row's
// last position) re-read s_last, which stays in cache.
template <bool FP8, bool PAGED, bool NT>
__device__ __forceinline__ void issue_group_loads(uint8_t *slot, const uint8_t *__restrict__ k,
                                                  const float *__restrict__ k_scale, int64_t row0,
                                                  int last, const DmaLane<FP8> &dl, int lane) {
  using C = IdxCfg<FP8>;
  const uint8_t *gbase = k + row0 * C::kRowBytes;
  if (last == C::kKeys - 1) {            // the whole group lies inside the row
#pragma unroll
    for (int j = 0; j < DmaLane<FP8>::kJ; ++j) dma16<NT>(gbase + dl.byte[j], slot + 1024 * j);
    if constexpr (FP8) dma4(k_scale + row0 + min(lane, C::kKeys - 1), slot + C::kGroupBytes);
  } else {
#pragma unroll
    for (int j = 0; j < DmaLane<FP8>::kJ; ++j)
      dma16<NT>(gbase + dl.byte[j] + (min(dl.key[j], last) - dl.key[j]) * C::kRowBytes,
                slot + 1024 * j);
    if constexpr (FP8) dma4(k_scale + row0 + min(lane, last), slot + C::kGroupBytes);
  }
}
template <bool FP8, bool PAGED>
__device__ __forceinline__ void issue_group(uint8_t *slot, const uint8_t *__restrict__ k,
                                            const float *__restrict__ k_scale, int64_t base_row,
                                            int page, int64_t s0, int64_t s_last,
                                            const DmaLane<FP8> &dl, int lane, bool cached) {
  const int64_t row0 = PAGED ? (int64_t)page * kPage + (s0 & 63) : base_row + s0;
  const int last = min((int)(s_last - s0), IdxCfg<FP8>::kKeys - 1);   // last valid key offset
  if (cached)
    issue_group_loads<FP8, PAGED, false>(slot, k, k_scale, row0, last, dl, lane);
  else
    issue_group_loads<FP8, PAGED, true>(slot, k, k_scale, row0, last, dl, lane);
}

// MFMA + fused epilogue for the group in `slot`; returns in lane (g, c) the score of key
// 16g + c of the group (for bf16 only lanes with g < 2 carry one).
template <bool FP8>
__device__ __forceinline__ float consume_group(const uint8_t *slot,
                                               const i32x4 (&qf)[4][IdxCfg<FP8>::kChunks],
                                               const HeadWeights &hw, int lane) {
  using C = IdxCfg<FP8>;
  const int c = lane & 15, g = lane >> 4;
  float mine = 0.f;
#pragma unroll
  for (int u = 0; u < C::kTiles; ++u) {
    const int key = 16 * u + c;
    i32x4 kf[C::kChunks];
#pragma unroll
    for (int i = 0; i < C::kChunks; ++i) {
      const int chunk = (g * C::kChunks + i) ^ key_swz<FP8>(key);
      kf[i] = *reinterpret_cast<const i32x4 *>(slot + key * C::kRowBytes + 16 * chunk);
    }
    f32x4 acc[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (FP8) {
        const i32x8 a = __builtin_shufflevector(qf[hb][0], qf[hb][1], 0, 1, 2, 3, 4, 5, 6, 7);
        const i32x8 bb = __builtin_shufflevector(kf[0], kf[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, acc[hb], 0, 0, 0, 127, 0, 127);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[hb][t]),
                                                            __builtin_bit_cast(bf16x8, kf[t]),
                                                            acc[hb], 0, 0, 0);
      }
    }
    const float v = head_sum(acc, hw);   // all 64 heads of key c, in every lane (., c)
    if (g == u) mine = v;
  }
  if constexpr (FP8) mine *= reinterpret_cast<const float *>(slot + C::kGroupBytes)[lane];
  return mine;
}

// HIST: also count the scores of the workgroup by the 12-bit leading digit of their order
// keys (the first stage of the few-row top-k) and deposit the nonzero bins, compressed, as
// list blockIdx.x of row r.
template <bool FP8, bool PAGED, bool HIST>
__global__ __launch_bounds__(IdxCfg<FP8>::kWaves * kWave) void indexer_mfma_kernel(
    RowsDev rows, int R, const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, const float *__restrict__ w,
    float *__restrict__ logits, int64_t ld, uint32_t *__restrict__ hcnt,
    uint32_t *__restrict__ hlist, int hstride, int cached) {
  using C = IdxCfg<FP8>;
  constexpr int kQChunks = kIdxHeads * C::kRowBytes / 16;
  constexpr int kThreads = C::kWaves * kWave;
  extern __shared__ __attribute__((aligned(16))) uint8_t idx_smem[];
  uint8_t *smem = idx_smem;
  i32x4 *q_lds = reinterpret_cast<i32x4 *>(smem);
  uint32_t *hist = reinterpret_cast<uint32_t *>(smem + kQChunks * 16 + C::kWaves * C::kDepth * C::kSlotBytes);
  const int r = grid_row();
  if (r >= R) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r];
  // The row's key groups are dealt to its waves round-robin (wave wr of WR takes groups wr,
  // wr + WR, ...), so at any time the row's waves stream one contiguous window of it.
  const int n_row_groups = (len + C::kKeys - 1) / C::kKeys;
  const int waves_per_row = gridDim.x * C::kWaves;
  const int wr = blockIdx.x * C::kWaves + wave;
  if (blockIdx.x * C::kWaves >= n_row_groups) {
    if (HIST && threadIdx.x == 0) hcnt[(size_t)r * hstride + blockIdx.x] = 0;
    return;
  }
  const bool active = wr < n_row_groups;
  const int n_groups = active ? (n_row_groups - wr + waves_per_row - 1) / waves_per_row : 0;
  const int64_t s_last = len - 1;
  const int b = rows.row_seq[r];
  uint8_t *ring = smem + kQChunks * 16 + wave * C::kDepth * C::kSlotBytes;
  int64_t base_row = 0;
  int page_lane = 0;   // paged layout: lane j holds the page of the wave's j-th group
  DmaLane<FP8> dl;
  // loads per group: kGroupBytes/1024 key instructions (+1 scale instruction for fp8)
  constexpr int kLoads = C::kGroupBytes / 1024 + (FP8 ? 1 : 0);
  auto group_start = [&](int j) { return (int64_t)(wr + j * waves_per_row) * C::kKeys; };
  auto group_page = [&](int j) {
    return PAGED ? __builtin_amdgcn_readlane(page_lane, j) : 0;
  };
  if (active) {
    if constexpr (PAGED) {
      if (lane < n_groups)
        page_lane = rows.page_table[(int64_t)b * rows.max_pages + (group_start(lane) >> 6)];
    } else {
      base_row = rows.seq_start[b];
    }
    // the first C::kDepth-1 key groups start streaming before the query block is loaded
    dl.init(lane);
    const int n_pro = min(C::kDepth - 1, n_groups);
    for (int d = 0; d < n_pro; ++d)
      issue_group<FP8, PAGED>(ring + d * C::kSlotBytes, k, k_scale, base_row, group_page(d),
                              group_start(d), s_last, dl, lane, cached);
  }
  if constexpr (HIST)
    for (int i = threadIdx.x; i < kLeadBins; i += kThreads) hist[i] = 0;
  {
    const i32x4 *qg = reinterpret_cast<const i32x4 *>(q + (int64_t)r * kIdxHeads * C::kRowBytes);
    for (int i = threadIdx.x; i < kQChunks; i += kThreads) q_lds[i] = qg[i];
  }
  __syncthreads();

  if (active) {
    // q operand of head 16*hb + c, dims [32g, 32g+32) (fp8) / [64g, 64g+64) (bf16)
    i32x4 qf[4][C::kChunks];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int i = 0; i < C::kChunks; ++i)
        qf[hb][i] = q_lds[(hb * 16 + c) * (C::kRowBytes / 16) + g * C::kChunks + i];
    // head weights of the result rows this lane holds: heads 16*hb + 4g + i
    float wt[4][4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t hj = (int64_t)r * kIdxHeads + hb * 16 + 4 * g + i;
        wt[hb][i] = FP8 ? w[hj] * q_scale[hj] : w[hj];
      }
    const HeadWeights hw = head_weights(wt);
    float *out = logits + (int64_t)r * ld;
    for (int i = 0; i < n_groups; ++i) {
      if (i + C::kDepth - 1 < n_groups) {
        issue_group<FP8, PAGED>(ring + ((i + C::kDepth - 1) % C::kDepth) * C::kSlotBytes, k, k_scale,
                                base_row, group_page(i + C::kDepth - 1), group_start(i + C::kDepth - 1),
                                s_last, dl, lane, cached);
        // group i is older than the C::kDepth-1 groups issued after it and than the score
        // stores of the iterations since it was issued (one per iteration: every group holds a
        // valid key); vector memory completes in order, and stores count too
        if (i >= C::kDepth - 1) __builtin_amdgcn_s_waitcnt(vmcnt_only((kLoads + 1) * (C::kDepth - 1)));
        else __builtin_amdgcn_s_waitcnt(vmcnt_only(kLoads * (C::kDepth - 1)));
      } else {
        // tail: nothing is issued past the wave's groups, so wait for every load in flight
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      }
      const float v = consume_group<FP8>(ring + (i % C::kDepth) * C::kSlotBytes, qf, hw, lane);
      const int64_t s = group_start(i) + lane;
      if (lane < C::kKeys && s < len) {
        out[s] = v;
        if constexpr (HIST) atomicAdd(&hist[order_key(v) >> (32 - kLeadDigitBits)], 1u);
      }
    }
  }

  if constexpr (HIST) {
    __syncthreads();   // every wave's counts are in (waves without groups come straight here)
    // ordered compaction of the nonzero bins: thread t owns bins PER*t .. PER*t+PER-1
    constexpr int PER = kLeadBins / kThreads;
    uint32_t nz = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) nz += hist[PER * threadIdx.x + j] ? 1u : 0u;
    uint32_t inc = nz;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t u = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += u;
    }
    // wave totals go to the query block area: every wave holds its q operands in registers
    uint32_t *wtot = reinterpret_cast<uint32_t *>(q_lds);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t off = inc - nz, total = 0;
    for (int wv = 0; wv < C::kWaves; ++wv) {
      off += (wv < wave) ? wtot[wv] : 0u;
      total += wtot[wv];
    }
    uint32_t *dst = hlist + ((size_t)r * hstride + blockIdx.x) * kLeadBins;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t bin = PER * threadIdx.x + j, cnt = hist[bin];
      if (cnt) dst[off++] = (bin << 16) | cnt;
    }
    if (threadIdx.x == 0) hcnt[(size_t)r * hstride + blockIdx.x] = total;
  }
}

size_t indexer_lds_bytes(bool fp8, bool hist) {
  using F = IdxCfg<true>;
  using B = IdxCfg<false>;
  const size_t base = fp8 ? (size_t)kIdxHeads * F::kRowBytes + (size_t)F::kWaves * F::kDepth * F::kSlotBytes
                          : (size_t)kIdxHeads * B::kRowBytes + (size_t)B::kWaves * B::kDepth * B::kSlotBytes;
  return base + (hist ? sizeof(uint32_t) * kLeadBins : 0);
}

template <bool FP8, bool PAGED, bool HIST>
static hipError_t launch_one(dim3 grid, size_t shm, hipStream_t stream, const RowsDev &rows,
                             int R, const uint8_t *q8, const float *q_scale, const uint8_t *k8,
                             const float *k_scale, const float *w, float *logits, int64_t ld,
                             uint32_t *hcnt, uint32_t *hlist, int hstride, int cached) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(&indexer_mfma_kernel<FP8, PAGED, HIST>, (int)shm, lds_set);
  if (e != hipSuccess) return e;
  indexer_mfma_kernel<FP8, PAGED, HIST><<<grid, IdxCfg<FP8>::kWaves * kWave, shm, stream>>>(
      rows, R, q8, q_scale, k8, k_scale, w, logits, ld, hcnt, hlist, hstride, cached);
  return hipGetLastError();
}

// One workgroup per CU at a time (the LDS rings fill most of the CU's 160 KB); the keys per
// wave are sized for about DSA_IDX_BLOCKS workgroups in all, whole 64-key multiples.
static int64_t keys_per_wave(int num_rows, int max_row_len, bool fp8) {
  const int64_t total = (int64_t)num_rows * max_row_len;
  constexpr int64_t kBlocksTarget = DSA_IDX_BLOCKS;
  const int64_t waves = fp8 ? IdxCfg<true>::kWaves : IdxCfg<false>::kWaves;
  int64_t kpw = (total + waves * kBlocksTarget - 1) / (waves * kBlocksTarget);
  kpw = ((kpw + 63) / 64) * 64;
  if (kpw < 64) kpw = 64;
  // at most 64 groups per wave (one page id per lane)
  const int64_t max_kpw = 64 * (fp8 ? IdxCfg<true>::kKeys : IdxCfg<false>::kKeys);
  return kpw > max_kpw ? max_kpw : kpw;
}

int indexer_blocks_per_row(int num_rows, int max_row_len, bool fp8) {
  const int64_t per_block = (fp8 ? IdxCfg<true>::kWaves : IdxCfg<false>::kWaves) *
                            keys_per_wave(num_rows, max_row_len, fp8);
  return (int)((max_row_len + per_block - 1) / per_block);
}

template <bool HIST>
static hipError_t launch_indexer(const RowsHost &rh, bool paged, bool fp8, const void *q,
                                 const float *q_scale, const void *k, const float *k_scale,
                                 const float *w, float *logits, int64_t ld, uint32_t *hcnt,
                                 uint32_t *hlist, int hstride, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  const dim3 grid = row_grid((unsigned)indexer_blocks_per_row(rh.num_rows, rh.max_row_len, fp8),
                             rh.num_rows);
  const size_t shm = indexer_lds_bytes(fp8, HIST);
  const uint8_t *q8 = static_cast<const uint8_t *>(q);
  const uint8_t *k8 = static_cast<const uint8_t *>(k);
  const int cached = rh.num_rows > rh.num_seqs;   // rows share sequences: keep keys in cache
  if (fp8)
    return paged ? launch_one<true, true, HIST>(grid, shm, stream, rows, rh.num_rows, q8, q_scale, k8, k_scale, w, logits, ld, hcnt, hlist, hstride, cached)
                 : launch_one<true, false, HIST>(grid, shm, stream, rows, rh.num_rows, q8, q_scale, k8, k_scale, w, logits, ld, hcnt, hlist, hstride, cached);
  return paged ? launch_one<false, true, HIST>(grid, shm, stream, rows, rh.num_rows, q8, q_scale, k8, k_scale, w, logits, ld, hcnt, hlist, hstride, cached)
               : launch_one<false, false, HIST>(grid, shm, stream, rows, rh.num_rows, q8, q_scale, k8, k_scale, w, logits, ld, hcnt, hlist, hstride, cached);
}

hipError_t launch_indexer_mfma(const RowsHost &rh, bool paged, bool fp8, const void *q,
                               const float *q_scale, const void *k, const float *k_scale,
                               const float *w, float *logits, int64_t ld, hipStream_t stream) {
  return launch_indexer<false>(rh, paged, fp8, q, q_scale, k, k_scale, w, logits, ld, nullptr,
                               nullptr, 0, stream);
}

hipError_t launch_indexer_mfma_hist(const RowsHost &rh, bool paged, bool fp8, const void *q,
                                    const float *q_scale, const void *k, const float *k_scale,
                                    const float *w, float *logits, int64_t ld,
                                    const TopkHistDest &hist, hipStream_t stream) {
  return launch_indexer<true>(rh, paged, fp8, q, q_scale, k, k_scale, w, logits, ld, hist.hcnt,
                              hist.hlist, hist.stride, stream);
}

}  // namespace dsa
