// indexer_core.h -- the key-streaming core of the lightning indexer on gfx950, shared by the
// indexer kernels and the one-launch decode kernel.
//
// I[t,s] = sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:]) over the preceding tokens s of the query's
// sequence ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ① Lightning Indexer: a few indexer
// heads, one key per token shared by all heads, FP8 supported).
//
// Decode-shaped work is bound by the key stream from HBM: every key byte is read once and
// meets 64 heads (64 flop/B in bf16, 128 flop/B in fp8), far under the MFMA ridge.  A row's
// keys are cut into 4 KB groups (32 fp8 or 16 bf16 keys); each wave streams its groups
// through a private ring of DEPTH LDS slots filled by direct global->LDS loads (keys never
// pass through VGPRs, DEPTH-1 groups are in flight while one is multiplied), keeps the row's
// 64x128 query block resident in registers as MFMA operands, and fuses ReLU, the head
// weights, the fp8 scales and the 64-head sum into the MFMA epilogue.
//
// Per 16-key tile a wave forms the 64 heads x 16 keys scores with the keys as the N
// dimension of 16x16 MFMA tiles (4 head blocks of 16), K = the 128 dims: lane (g, c) holds
// dims [32g, 32g+32) (fp8) / [64g, 64g+64) (bf16) of key c as the B operand and the same dims
// of head 16 hb + c as the A operand.
//   bf16: 4 x v_mfma_f32_16x16x32_bf16 per head block;  fp8: 1 x
//   v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales).
// Epilogue: ReLU and the head weights w' (w * q_scale for fp8) summed over the 64 heads by two
// bf16 MFMAs (head_sum); fp8 then multiplies by the key's scale.
#pragma once
#include "dsa_device.h"

namespace dsa {

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;

template <bool FP8>
struct IdxKeys {
  static constexpr int kRowBytes = kIdxDim * (FP8 ? 1 : 2);   // 128 / 256
  static constexpr int kGroupBytes = 4096;
  static constexpr int kKeys = kGroupBytes / kRowBytes;        // keys per group: 32 / 16
  static constexpr int kTiles = kKeys / 16;                    // 16-key MFMA tiles per group
  static constexpr int kChunks = kRowBytes / 64;               // 16-byte chunks per lane per key
  static constexpr int kSlotBytes = kGroupBytes + (FP8 ? 256 : 0);   // keys (+ their scales)
  static constexpr int kQBytes = kIdxHeads * kRowBytes;        // the row's query block
  static constexpr int kLoads = kGroupBytes / 1024 + (FP8 ? 1 : 0);   // DMA instructions per group
};

// Shape of a workgroup of the streaming core: WAVES waves with rings of DEPTH slots.  LDS:
// the query block, then the rings (the head weights and query scales go to a 512-byte
// buffer of the caller's).
template <bool FP8, int WAVES, int DEPTH>
struct IdxShape : IdxKeys<FP8> {
  static constexpr int kWaves = WAVES;
  static constexpr int kDepth = DEPTH;
  static constexpr int kThreads = WAVES * kWave;
  static constexpr int kRingBytes = WAVES * DEPTH * IdxKeys<FP8>::kSlotBytes;
  static constexpr int kCoreBytes = IdxKeys<FP8>::kQBytes + kRingBytes;
  static_assert(DEPTH >= 2 && DEPTH <= 4, "one to three groups in flight");
};

// XOR applied to the 16-byte chunk index of key `key` inside a slot (low 3 bits for 128-byte
// fp8 rows, low 4 bits for 256-byte bf16 rows): 16 consecutive keys read at one logical chunk
// land on 16 distinct 16-byte bank groups.  Applied on the global side, by choosing which
// chunk each lane fetches.
template <bool FP8>
__device__ __forceinline__ int key_swz(int key) {
  if constexpr (FP8) return ((key >> 1) & 7) ^ ((key & 1) << 2);
  return key & 15;
}

// Global->LDS loads of 16 (keys) and 4 (scales, weights) bytes per lane: lane l lands at
// lds + l * size.  Keys read once carry the non-temporal hint, which keeps the scores and the
// attention's cache lines in L2 and the Infinity Cache for the later stages (measured: plain
// loads cost 3 to 10 us per decode step); keys that several rows of one sequence read at about
// the same time (multi-token decode) are loaded plainly and hit in L2 for the later rows.
// Written as two-instruction asm statements rather than the builtin: the compiler treats every
// LDS write it cannot disambiguate from a pending global->LDS load as aliasing it and would
// wait for all of them first (draining the rings).  The instructions write no register and
// consume their operands at issue; the waits for the data use explicit vmcnt counts (loads
// complete in order).
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
}
template <bool NT>
__device__ __forceinline__ void key_dma16(const void *g, void *lds) {
  if constexpr (NT)
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g),
                     "s"(lds_addr(lds))
                     : "memory");
  else
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                     "s"(lds_addr(lds))
                     : "memory");
}
__device__ __forceinline__ void key_dma4(const void *g, void *lds) {
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(lds))
                   : "memory");
}

// Per-lane constant part of a group's DMA addresses: for key instruction j, the key of the
// group this lane's 16 bytes belong to and the byte offset of its source chunk.
template <bool FP8>
struct DmaLane {
  static constexpr int kJ = IdxKeys<FP8>::kGroupBytes / 1024;
  int key[kJ];
  int byte[kJ];
  __device__ __forceinline__ void init(int lane) {
    using C = IdxKeys<FP8>;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int pos = 1024 * j + 16 * lane;             // byte position inside the slot
      key[j] = pos / C::kRowBytes;
      const int chunk = (pos % C::kRowBytes) >> 4;      // physical chunk
      byte[j] = key[j] * C::kRowBytes + 16 * (chunk ^ key_swz<FP8>(key[j]));
    }
  }
};

// Issues the loads of the key group whose first key is cache row row0 into `slot`; `last` is
// the offset of the group's last valid key (keys past it re-read it, which stays in cache).
template <bool FP8, bool NT>
__device__ __forceinline__ void issue_group_loads(uint8_t *slot, const uint8_t *__restrict__ k,
                                                  const float *__restrict__ k_scale, int64_t row0,
                                                  int last, const DmaLane<FP8> &dl, int lane) {
  using C = IdxKeys<FP8>;
  const uint8_t *gbase = k + row0 * C::kRowBytes;
  if (last == C::kKeys - 1) {            // the whole group lies inside the row
#pragma unroll
    for (int j = 0; j < DmaLane<FP8>::kJ; ++j) key_dma16<NT>(gbase + dl.byte[j], slot + 1024 * j);
    if constexpr (FP8) key_dma4(k_scale + row0 + min(lane, C::kKeys - 1), slot + C::kGroupBytes);
  } else {
#pragma unroll
    for (int j = 0; j < DmaLane<FP8>::kJ; ++j)
      key_dma16<NT>(gbase + dl.byte[j] + (min(dl.key[j], last) - dl.key[j]) * C::kRowBytes,
                    slot + 1024 * j);
    if constexpr (FP8) key_dma4(k_scale + row0 + min(lane, last), slot + C::kGroupBytes);
  }
}
// base_row: contiguous layout, cache row of position 0; paged layout: page holds the cache
// page of the group (a group never crosses a 64-token page).
template <bool FP8, bool PAGED>
__device__ __forceinline__ void issue_group(uint8_t *slot, const uint8_t *__restrict__ k,
                                            const float *__restrict__ k_scale, int64_t base_row,
                                            int page, int64_t s0, int64_t s_last,
                                            const DmaLane<FP8> &dl, int lane, bool cached) {
  const int64_t row0 = PAGED ? (int64_t)page * kPage + (s0 & 63) : base_row + s0;
  const int last = min((int)(s_last - s0), IdxKeys<FP8>::kKeys - 1);   // last valid key offset
  if (cached)
    issue_group_loads<FP8, false>(slot, k, k_scale, row0, last, dl, lane);
  else
    issue_group_loads<FP8, true>(slot, k, k_scale, row0, last, dl, lane);
}

// MFMA + fused epilogue for the group in `slot`; returns in lane (g, c) the score of key
// 16g + c of the group (for bf16 only lanes with g < 2 carry one).
template <bool FP8>
__device__ __forceinline__ float consume_group(const uint8_t *slot,
                                               const i32x4 (&qf)[4][IdxKeys<FP8>::kChunks],
                                               const HeadWeights &hw, int lane) {
  using C = IdxKeys<FP8>;
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

// Waits until at most n vector-memory operations of this wave are outstanding (n < 4: the
// number of prologue groups issued after the row data).
template <int LOADS>
__device__ __forceinline__ void wait_row_data(int groups_after) {
  if (groups_after >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_only(3 * LOADS));
  else if (groups_after == 2) __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * LOADS));
  else if (groups_after == 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(LOADS));
  else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

// One workgroup's share of row r: wave `wave` scores the key groups g0 + j * gstride
// (j < ng), handing the score v of every valid position s to put(s, v) (lanes < kKeys).
// Every wave of the workgroup calls it (ng may be 0): it holds workgroup barriers.
// smem: S::kCoreBytes of LDS (query block, then the rings); wbuf: 512 bytes of LDS for the
// head weights and query scales, free for put() once the groups stream.  PUT_VMEM: put issues
// one vector-memory store per group (counted in the ring waits).  cached: plain key loads
// instead of non-temporal ones.
template <bool FP8, bool PAGED, int WAVES, int DEPTH, bool PUT_VMEM, class Put>
__device__ __forceinline__ void index_groups(uint8_t *smem, const RowsDev &rows, int r,
                                             const uint8_t *__restrict__ q,
                                             const float *__restrict__ q_scale,
                                             const uint8_t *__restrict__ k,
                                             const float *__restrict__ k_scale,
                                             const float *__restrict__ w, uint8_t *wbuf,
                                             int64_t g0, int64_t gstride, int ng, bool cached,
                                             Put put) {
  using S = IdxShape<FP8, WAVES, DEPTH>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r];
  const int64_t s_last = len - 1;
  const int b = rows.row_seq[r];
  uint8_t *row_data = smem;
  uint8_t *ring = smem + S::kQBytes + wave * DEPTH * S::kSlotBytes;
  // the row data first: query block (1 KB per instruction, dealt to the waves), head weights
  // and query scales (256 B each, the last two waves)
  constexpr int kQInstr = S::kQBytes / 1024;
  const uint8_t *qrow = q + (int64_t)r * S::kQBytes;
  for (int j = wave; j < kQInstr; j += WAVES)
    key_dma16<false>(qrow + 1024 * j + 16 * lane, row_data + 1024 * j);
  if (wave == WAVES - 1) key_dma4(w + (int64_t)r * kIdxHeads + lane, wbuf);
  if (FP8 && wave == WAVES - 2) key_dma4(q_scale + (int64_t)r * kIdxHeads + lane, wbuf + 256);
  // then the first DEPTH-1 key groups
  int64_t base_row = 0;
  int page_lane = 0;   // paged layout: lane j holds the page of the wave's j-th group
  DmaLane<FP8> dl;
  auto group_start = [&](int j) { return (g0 + j * gstride) * S::kKeys; };
  auto group_page = [&](int j) { return PAGED ? __builtin_amdgcn_readlane(page_lane, j) : 0; };
  const int n_pro = min(DEPTH - 1, ng);
  if (ng > 0) {
    if constexpr (PAGED) {
      if (lane < ng)
        page_lane = rows.page_table[(int64_t)b * rows.max_pages + (group_start(lane) >> 6)];
    } else {
      base_row = rows.seq_start[b];
    }
    dl.init(lane);
    for (int d = 0; d < n_pro; ++d)
      issue_group<FP8, PAGED>(ring + d * S::kSlotBytes, k, k_scale, base_row, group_page(d),
                              group_start(d), s_last, dl, lane, cached);
  }
  // this wave's share of the row data has landed (the key groups stay in flight)
  wait_row_data<S::kLoads>(n_pro);
  lds_barrier();

  // q operand of head 16*hb + c, dims [32g, 32g+32) (fp8) / [64g, 64g+64) (bf16)
  const i32x4 *q_lds = reinterpret_cast<const i32x4 *>(row_data);
  i32x4 qf[4][S::kChunks];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < S::kChunks; ++i)
      qf[hb][i] = q_lds[(hb * 16 + c) * (S::kRowBytes / 16) + g * S::kChunks + i];
  // head weights of the result rows this lane holds: heads 16*hb + 4g + i
  const float *w_lds = reinterpret_cast<const float *>(wbuf);
  const float *qs_lds = reinterpret_cast<const float *>(wbuf + 256);
  float wt[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb * 16 + 4 * g + i;
      wt[hb][i] = FP8 ? w_lds[h] * qs_lds[h] : w_lds[h];
    }
  const HeadWeights hw = head_weights(wt);
  // every wave holds its weights before put() may reuse wbuf
  lds_barrier();
  if (ng == 0) return;
  constexpr int L = S::kLoads;
  for (int i = 0; i < ng; ++i) {
    if (i + DEPTH - 1 < ng) {
      issue_group<FP8, PAGED>(ring + ((i + DEPTH - 1) % DEPTH) * S::kSlotBytes, k, k_scale,
                              base_row, group_page(i + DEPTH - 1), group_start(i + DEPTH - 1),
                              s_last, dl, lane, cached);
      // group i is older than the DEPTH-1 groups issued after it and, with PUT_VMEM, than the
      // score stores of the iterations since it was issued (one per iteration: every group
      // holds a valid key); vector memory completes in order, and stores count too
      if (PUT_VMEM && i >= DEPTH - 1) __builtin_amdgcn_s_waitcnt(vmcnt_only((L + 1) * (DEPTH - 1)));
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(L * (DEPTH - 1)));
    } else {
      // tail: nothing is issued past the wave's groups, so wait for every load in flight
      __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    }
    const float v = consume_group<FP8>(ring + (i % DEPTH) * S::kSlotBytes, qf, hw, lane);
    const int64_t s = group_start(i) + lane;
    if (lane < S::kKeys && s < len) put(s, v);
  }
}

}  // namespace dsa
