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
// bf16 kernel design.  A workgroup owns one query row, all 128 heads (8 waves x 16 heads)
// and a range of its top-k slots.  The cache rows of the valid slots are resolved and
// compacted up front; the selected entries are then gathered 32 at a time straight into a
// ring of LDS tiles with global->LDS loads (several tiles in flight, no staging registers),
// a swizzle of the 16-byte chunks applied through the choice of source chunk.  Each wave
// computes the transposed score tile S^T = C . Q^T (entries as MFMA rows, its 16 heads as
// columns, q resident in registers), runs the online softmax in fp32 in the log2 domain, and
// accumulates O^T += V^T . P^T with V read from the same LDS tile through the gfx950
// transposing LDS read (ds_read_b64_tr_b16), so the tile is stored once, row-major, for
// both products.  Few-row (decode) batches split the slots over several workgroups; each
// writes a normalised bf16 partial and its log-sum-exp, and a combine kernel merges them.
// When a split batch is small enough (at most 256 workgroups either way), each (row, split)
// gets two workgroups of 64 heads: four waves own the heads and four only share the
// selection and the tile loads, so each CU moves half the query block and the tile loop
// carries half the products.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "topk_select.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path: one workgroup per (row, head), two passes over the selected entries.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void mla_f32_kernel(RowsDev rows, int R, int H, int Dqk, int Dv,
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
  const int h = blockIdx.x, r = grid_row();
  if (r >= R) return;
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
  const dim3 grid = row_grid(H, rh.num_rows);
  const size_t shm = sizeof(float) * ((k + 1) & ~1) + sizeof(int64_t) * k + sizeof(float) * Dqk;
  if (paged)
    mla_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, rh.num_rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                     lse);
  else
    mla_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, rh.num_rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                      lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// bf16 MFMA path, d_qk = 576 (512 latent + 64 RoPE), d_v = 512.
// ------------------------------------------------------------------------------------
#ifndef DSA_MLA_QK_PREFETCH
#define DSA_MLA_QK_PREFETCH 2
#endif
#ifndef DSA_MLA_PV_PREFETCH
#define DSA_MLA_PV_PREFETCH 3
#endif
#ifndef DSA_MLA_HEAD_GROUPS
#define DSA_MLA_HEAD_GROUPS 2
#endif
#ifndef DSA_MLA_DEPTH
#define DSA_MLA_DEPTH 4
#endif
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;          // 1152 B per cache entry
constexpr int kTile = 32;                    // entries per LDS tile
constexpr int kTileBytes = kTile * kRowBytes;   // 36 KB = 36 DMA instructions of 1 KB
constexpr int kMlaWaves = 8;                 // 16 heads each
constexpr int kMlaThreads = kMlaWaves * kWave;
constexpr int kHeadsPerBlock = 128;
constexpr int kMlaHeadGroups = DSA_MLA_HEAD_GROUPS;   // 1 or 2
constexpr int kRing = DSA_MLA_DEPTH;          // LDS tile slots (kRing - 1 tiles in flight)
constexpr int kMaxSlotsPerSplit = 2048;
constexpr int kSlotRounds = kMaxSlotsPerSplit / kMlaThreads;   // 4
static_assert(kTileBytes % 1024 == 0, "tile DMA is whole 1 KB instructions");

// XOR swizzle of the 16-byte chunk index inside its aligned group of 8 chunks: bit 0 =
// row bit 0 ^ row bit 3, bit 1 = row bit 1 ^ row bit 3, bit 2 = row bit 1.  Picked by
// measuring LDS read throughput on gfx950 over all swizzles built from row bits {0,1,3,4}:
// with it the score-operand loads (16 rows 8a + b, a 16-byte chunk each) run at the rate
// of contiguous loads, and the transposing value loads at the best rate found.  Row bit 2
// is unused: rows r and r + 4 share the swizzle.
__device__ __forceinline__ int swz(int row) {
  return ((row ^ (row >> 3)) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1) | (((row >> 1) & 1) << 2);
}

typedef bf16x4 __attribute__((address_space(3))) *lds_bf16x4_ptr;
typedef void __attribute__((address_space(3))) *lds_void_ptr;

constexpr int vmcnt_only(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

struct MlaShared {
  uint8_t tiles[kRing][kTileBytes];
  uint32_t crow[kMaxSlotsPerSplit];        // cache rows of the split's valid slots, compacted
  uint32_t wcount[kMlaWaves];
  uint32_t wbad[kMlaWaves];                // invalid slots seen by each wave
};

// The 36 DMA instructions of a tile go to waves 0..7 in turn (waves 0-3 issue 5, 4-7
// issue 4).  LDS position P = 1024*j + 16*lane of the tile holds entry P / 1152,
// physical chunk (P % 1152) / 16, i.e. logical chunk physical ^ swz(entry).
constexpr int kTileDma = kTileBytes / 1024;   // 36
constexpr int kDmaMax = (kTileDma + kMlaWaves - 1) / kMlaWaves;   // 5
// One 16-byte-per-lane global->LDS load (1 KB per wave at `lds`, lane l at lds + 16 l).
// Written as a two-instruction asm statement rather than the builtin: the compiler treats
// every LDS access it cannot disambiguate from a pending global->LDS load as aliasing it
// and, before the transposing LDS reads of the value product, would wait for all such
// loads, draining the tile ring each iteration.  The instruction writes no register, its
// operands are consumed at issue, and the kernel waits for the data with explicit vmcnt
// counts (loads complete in order) before any wave reads the tile.
__device__ __forceinline__ void dma16(const void *src, const void *lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(la)
                   : "memory");
}

__device__ __forceinline__ int tile_dma_count(int wave) {
  return kTileDma / kMlaWaves + (wave < kTileDma % kMlaWaves ? 1 : 0);
}
// Per-lane constants of a wave's DMA instructions, two 16-bit fields per word: for
// instruction i, (tile entry) | (byte offset of the source chunk inside the entry) << 5.
struct TileDma {
  uint32_t pk[(kDmaMax + 1) / 2];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int w = 0; w < (kDmaMax + 1) / 2; ++w) pk[w] = 0;
#pragma unroll
    for (int i = 0; i < kDmaMax; ++i) {
      const int pos = 1024 * (wave + kMlaWaves * i) + 16 * lane;
      const int e = min(pos / kRowBytes, kTile - 1);   // instructions past the tile: unused
      const int byte = 16 * (((pos - e * kRowBytes) >> 4) ^ swz(e)) & 2047;
      pk[i >> 1] |= (uint32_t)(e | (byte << 5)) << (16 * (i & 1));
    }
  }
};
// The DMA instructions of one tile, prepared ahead: source addresses resolved from the
// tile's cache rows, issued one at a time where they do not stall the wave.
// Instruction i of a wave's tile loads reads, in each lane, tile entry entry(i) starting at
// byte offset byte(i) of the entry (both from the packed per-lane constants).
__device__ __forceinline__ uint32_t dma_field(const TileDma &td, int i) {
  // opaque copy: keeps the compiler from hoisting 64-bit addresses out of the tile loop
  uint32_t p = td.pk[i >> 1];
  __asm__ volatile("" : "+v"(p));
  return (p >> (16 * (i & 1))) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t dma_row(const uint32_t *crow_tile, const TileDma &td, int i) {
  return crow_tile[dma_field(td, i) & 31u];
}
__device__ __forceinline__ void dma_issue(int i, uint32_t cache_row, uint8_t *dst,
                                          const uint8_t *__restrict__ kv, const TileDma &td,
                                          int n_dma, int wave) {
  if (i < kDmaMax - 1 || n_dma == kDmaMax)
    dma16(kv + (uint64_t)cache_row * kRowBytes + (dma_field(td, i) >> 5),
          dst + 1024 * (wave + kMlaWaves * i));
}
__device__ __forceinline__ void issue_tile(uint8_t *dst, const uint32_t *crow_tile,
                                          const uint8_t *__restrict__ kv, const TileDma &td,
                                          int n_dma, int wave) {
  uint32_t cr[kDmaMax];
#pragma unroll
  for (int i = 0; i < kDmaMax; ++i) cr[i] = dma_row(crow_tile, td, i);
#pragma unroll
  for (int i = 0; i < kDmaMax; ++i) dma_issue(i, cr[i], dst, kv, td, n_dma, wave);
}

// Waits until at most `younger` tiles of N loads each (issued after the awaited one) are
// still in flight; vector-memory loads complete in issue order.
static_assert(kRing >= 3 && kRing <= 4, "at most two tiles in flight behind the current one");
template <int N>
__device__ __forceinline__ void wait_younger(int younger) {
  if (younger >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * N));
  else if (younger >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_only(N));
  else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
}

// Workgroup -> (row, split).  Workgroups are dealt to the 8 XCDs round-robin by id, so
// all splits of a row land on one XCD: their query block and partials share its L2.
// Without a split (many rows, one workgroup each) the rows are taken from the last to the
// first: in a prefill batch later positions select more entries, so the longest rows start
// first and the short ones fill the end of the grid.
// With G head groups a (row, split) has G workgroups, each over 128 / G of the heads.
struct MlaCoord { int r, split, group; };
__device__ __forceinline__ bool mla_coord(int bid, int R, int S, int G, MlaCoord &c) {
  const int x = bid & 7, j = bid >> 3;
  const int sg = S * G;
  c.r = (j / sg) * 8 + x;
  const int rem = j % sg;
  c.split = rem / G;
  c.group = rem - c.split * G;
  if (sg == 1) c.r = R - 1 - c.r;   // the grid holds 8 * ceil(R / 8) >= R workgroups
  return c.r >= 0 && c.r < R;
}

// Finishing the row's top-k inside the attention workgroups (see mla_bf16_kernel).
struct MlaSel {
  const float *logits;   // the score rows (fallback of degenerate rows)
  int64_t ld;
  MbWs ws;               // the chunked filter's survivors
  int chunks;            // 4096-score chunks of the longest row
};
constexpr size_t kSelScratchBytes = (sizeof(BlockScratch<kMlaThreads>) + 15) & ~(size_t)15;
constexpr size_t kSelKeyOff = kSelScratchBytes;
constexpr size_t kSelPosOff = kSelKeyOff + sizeof(uint32_t) * kSurvivorCap;
constexpr size_t kSelCoffOff = kSelPosOff + sizeof(int32_t) * kSurvivorCap;
constexpr size_t kSelListOff =
    (kSelCoffOff + sizeof(uint32_t) * (kMaxChunks + 1) + 15) & ~(size_t)15;
static_assert(kSelListOff + sizeof(int32_t) * kMaxSlotsPerSplit <= (size_t)kRing * kTileBytes,
              "selection scratch fits the tile ring");

// One workgroup: the heads of head group `group` (all 128, or 64 of them) of query row r over
// one split of its top-k slots.  Wave w owns heads group * 128 / HG + 16w .. +15 over the full
// contractions.  Per tile of 32 entries it
// forms S^T = C . Q^T (entries as MFMA rows, 2 blocks of 16 entries x its 16 heads, q in
// registers), runs the online softmax, and accumulates O^T += V^T . P^T over all 512
// value dims, V^T read from the same LDS tile with the transposing LDS read.  Entry rows
// of the score blocks are permuted (block kb, row 4g + i <-> entry 8g + 4kb + i) so that
// each lane's weights are exactly the B operand of the value product.
// SEL: the row's top-k is not given but finished here, from the survivors of the chunked
// top-k filter (every split of the row selects the row's k positions in its tile ring, which
// is free until the first tile load, keeps its own slots and writes them to idx as well).
//
// The leading arguments are the ones the prologue needs first (scalars and pointers, so
// the launch can preload them into registers).
template <bool PAGED, bool SEL, int HG>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    int R, int splits, int k, int slots_per_split, int32_t *__restrict__ idx,
    const uint16_t *__restrict__ q, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_len, const int64_t *__restrict__ seq_start,
    const int32_t *__restrict__ page_table, int max_pages, float scale_log2,
    const uint8_t *__restrict__ kv, uint16_t *__restrict__ out, float *__restrict__ lse,
    uint16_t *__restrict__ part_o, float *__restrict__ part_lse, MlaSel sel) {
  constexpr int H = kHeadsPerBlock;
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_smem[];
  MlaShared &sh = *reinterpret_cast<MlaShared *>(mla_smem);
  MlaCoord co;
  static_assert(HG == 1 || HG == 2, "one or two head groups");
  if (!mla_coord(blockIdx.x, R, splits, HG, co)) return;
  const int r = co.r, split = co.split;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  // waves below 8 / HG own 16 heads each; with two head groups waves 4-7 only take their
  // part in the selection and in the tile loads (one head group: a compile-time true)
  const bool mma = HG == 1 || wave < kMlaWaves / HG;
  const int h0 = co.group * (kHeadsPerBlock / HG) + (mma ? wave : 0) * 16;
  const int slot_begin = split * slots_per_split;
  const int n_slots = max(0, min(k, slot_begin + slots_per_split) - slot_begin);
  int32_t *idx_row = idx + (int64_t)r * k + slot_begin;   // read, or written when SEL

  // cache rows of the valid slots, compacted in slot order
  int n_valid = 0;
  bf16x8 qf[18];
  {
    int sv[kSlotRounds];
    // q^T operand: head h0 + c, dims 32t + 8g .. +8 (in flight during the slot resolution
    // and the first tile loads)
    auto load_q = [&]() {
      const bf16x8 *qp =
          reinterpret_cast<const bf16x8 *>(q + ((int64_t)r * H + h0 + c) * kDqk + 8 * g);
#pragma unroll
      for (int t = 0; t < 18; ++t) qf[t] = qp[4 * t];
    };
    if constexpr (SEL) {
      // the row's k positions, ascending, into the tile ring; slot j of the row is the j-th.
      // The query loads go out after the selection, whose loads they would hold up.
      const SurvivorLoads<kMlaThreads> sl = issue_survivor_loads<kMlaThreads>(sel.ws, r, sel.chunks);
      const int n = row_len[r];
      int32_t *lst = reinterpret_cast<int32_t *>(sh.tiles[0] + kSelListOff);
      if (n > k) {
        select_from_survivors<kMlaThreads>(
            sl, sel.logits, sel.ld, sel.ws, r, n, k, lst,
            *reinterpret_cast<BlockScratch<kMlaThreads> *>(sh.tiles[0]),
            reinterpret_cast<uint32_t *>(sh.tiles[0] + kSelKeyOff),
            reinterpret_cast<int32_t *>(sh.tiles[0] + kSelPosOff),
            reinterpret_cast<uint32_t *>(sh.tiles[0] + kSelCoffOff));
        __syncthreads();
      }
      if (mma) load_q();
#pragma unroll
      for (int j = 0; j < kSlotRounds; ++j) {
        const int t = j * kMlaThreads + threadIdx.x;
        const int slot = slot_begin + t;
        sv[j] = t < n_slots ? (n > k ? lst[slot] : (slot < n ? slot : -1)) : -1;
        if (t < n_slots && co.group == 0) idx_row[t] = sv[j];
      }
    } else {
      // the slot loads go out first (they need only the launch arguments), then the query
      // block, then the row's descriptor loads: waits on vector memory are in issue order,
      // so resolving the slots does not wait for the query block
#pragma unroll
      for (int j = 0; j < kSlotRounds; ++j) {
        const int t = j * kMlaThreads + threadIdx.x;
        sv[j] = t < n_slots ? idx_row[t] : -1;
      }
      __builtin_amdgcn_sched_barrier(0);
      if (mma) load_q();
    }
    __builtin_amdgcn_sched_barrier(0);
    const RowsDev rows{row_seq, row_len, seq_start, page_table, max_pages};
    const int len = row_len[r], b = row_seq[r];
    const int64_t seq_base = PAGED ? 0 : seq_start[b];
    int64_t crow_v[kSlotRounds];
    uint32_t bad = 0;
#pragma unroll
    for (int j = 0; j < kSlotRounds; ++j) {
      const int t = j * kMlaThreads + threadIdx.x;
      crow_v[j] = (sv[j] >= 0 && sv[j] < len)
                      ? (PAGED ? cache_row<PAGED>(rows, b, sv[j]) : seq_base + sv[j])
                      : -1;
      bad += (t < n_slots && crow_v[j] < 0) ? 1u : 0u;
    }
    // common case, every slot valid: the slots are their own compaction.  Each thread files
    // its slots' rows, wave 0 pads the last tile with slot 0's row, and one barrier settles
    // whether that stands.
#pragma unroll
    for (int j = 0; j < kSlotRounds; ++j) {
      const int t = j * kMlaThreads + threadIdx.x;
      if (t < n_slots) sh.crow[t] = (uint32_t)crow_v[j];
    }
    const int pad = ((n_slots + kTile - 1) / kTile) * kTile - n_slots;   // < kTile <= 64
    const uint32_t row0 = (uint32_t)__shfl((int)crow_v[0], 0, kWave);
    if (wave == 0 && lane < pad) sh.crow[n_slots + lane] = row0;
    const uint32_t wbad = (uint32_t)__popcll(__ballot(bad != 0));
    if (lane == 0) sh.wbad[wave] = wbad;
    lds_barrier();
    uint32_t any_bad = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) any_bad |= sh.wbad[w];
    if (any_bad == 0) n_valid = n_slots;
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < kSlotRounds; ++j) {
      if (any_bad == 0 || j * kMlaThreads >= n_slots) break;
      const bool ok = crow_v[j] >= 0;
      const uint64_t m = __ballot(ok);
      if (lane == 0) sh.wcount[wave] = (uint32_t)__popcll(m);
      lds_barrier();
      int before = n_valid, total = 0;
#pragma unroll
      for (int w = 0; w < kMlaWaves; ++w) {
        const int cw = (int)sh.wcount[w];
        before += w < wave ? cw : 0;
        total += cw;
      }
      if (ok) sh.crow[before + __popcll(m & lt)] = (uint32_t)crow_v[j];
      n_valid += total;
      lds_barrier();
    }
  }
  const int n_tiles = (n_valid + kTile - 1) / kTile;
  if (n_valid != n_slots) {
    // the tail of the last tile gathers a harmless valid row and is masked off
    if (threadIdx.x < n_tiles * kTile - n_valid) sh.crow[n_valid + threadIdx.x] = sh.crow[0];
    lds_barrier();
  }

  f32x4 oacc[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  const int n_dma = tile_dma_count(wave);
  TileDma td;
  td.init(wave, lane);
  // tile loads run kAhead tiles ahead of the tile being scored
  constexpr int kAhead = kRing - 1;
  for (int d = 0; d < kAhead && d < n_tiles; ++d)
    issue_tile(sh.tiles[d], sh.crow + d * kTile, kv, td, n_dma, wave);

  // score operand rows: block kb, lane row c <-> entry 8(c>>2) + (c&3) + 4kb (both share a
  // swizzle); dims 32t + 8g are chunk 4t + g: group t/2, in-group 4(t&1) + g
  const int arow = 8 * (c >> 2) + (c & 3);
  const int a_even = arow * kRowBytes + 16 * (g ^ swz(arow));
  const int a_odd = arow * kRowBytes + 16 * ((4 + g) ^ swz(arow));
  // value operand: transposing reads of entries 8g + tr_i (+4), dims 16nb + 4tr_q;
  // (chunk 2m + (tr_q >> 1)) ^ swz = 2 (m ^ (swz >> 1)) + ((tr_q >> 1) ^ (swz & 1))
  const int tr_i = c >> 2, tr_q = c & 3;
  const int swa = swz(8 * g + tr_i);
  const int ua = swa >> 1;
  const int v_off = (8 * g + tr_i) * kRowBytes + 8 * (tr_q & 1) + 16 * ((tr_q >> 1) ^ (swa & 1));

  // ---- scores of a tile: 18 steps of 32 dims, two independent 16-entry blocks; the operand
  // loads run kPf steps ahead of the products that use them
  auto scores = [&](const uint8_t *tile, f32x4 &sc0, f32x4 &sc1) {
    sc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    sc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kPf = DSA_MLA_QK_PREFETCH;
    bf16x8 xr[kPf][2];
#pragma unroll
    for (int t = 0; t < kPf; ++t) {
      const uint8_t *ap = tile + ((t & 1) ? a_odd : a_even) + 128 * (t >> 1);
      xr[t][0] = *reinterpret_cast<const bf16x8 *>(ap);
      xr[t][1] = *reinterpret_cast<const bf16x8 *>(ap + 4 * kRowBytes);
    }
#pragma unroll
    for (int t = 0; t < 18; ++t) {
      const bf16x8 x0 = xr[t % kPf][0], x1 = xr[t % kPf][1];
      if (t + kPf < 18) {
        const int tn = t + kPf;
        const uint8_t *ap = tile + ((tn & 1) ? a_odd : a_even) + 128 * (tn >> 1);
        xr[t % kPf][0] = *reinterpret_cast<const bf16x8 *>(ap);
        xr[t % kPf][1] = *reinterpret_cast<const bf16x8 *>(ap + 4 * kRowBytes);
      }
      // keep the scheduler from sinking the loads next to their use
      __builtin_amdgcn_sched_barrier(0);
      sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, qf[t], sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, qf[t], sc1, 0, 0, 0);
    }
  };
  // ---- online softmax of tile `it`: returns the bf16 weights (B operand of the value
  // product) and rescales the accumulators when the running maximum moves
  auto weights = [&](f32x4 sc0, f32x4 sc1, int it) {
    // only the last tile can hold padding entries: their scores become -inf
    const int nv = n_valid - it * kTile;
    if (nv < kTile) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (8 * g + i >= nv) sc0[i] = -INFINITY;
        if (8 * g + 4 + i >= nv) sc1[i] = -INFINITY;
      }
    }
    // tile maximum of head h0 + c in the scaled log2 domain (scale > 0; finite: the tile
    // has a valid entry)
    float mx = fmaxf(fmaxf(fmaxf(sc0[0], sc0[1]), fmaxf(sc0[2], sc0[3])),
                     fmaxf(fmaxf(sc1[0], sc1[1]), fmaxf(sc1[2], sc1[3])));
    mx = max_xor32(max_xor16(mx)) * scale_log2;
    // lazy online softmax (log2 domain): the reference maximum only moves when the tile
    // maximum exceeds it by more than 8, so weights stay <= 2^8 and rescales are rare
    const bool first = m_run == -INFINITY;
    const bool move = first || mx > m_run + 8.f;
    if (__ballot(move && !first)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
#pragma unroll
      for (int nb = 0; nb < 32; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] *= alpha;
      l_part *= alpha;
    }
    if (move) m_run = mx;
    const float neg_m = -m_run;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sc0[i], scale_log2, neg_m));
      p[4 + i] = __builtin_amdgcn_exp2f(fmaf(sc1[i], scale_log2, neg_m));
    }
    l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
  };
  // ---- O^T += V^T . P^T over a tile: value rows 16nb + c
  auto accumulate = [&](const uint8_t *tile, bf16x8 pf) {
    const uint8_t *va[4];   // per-lane bases; the 128-byte group and the +4 entries are immediates
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) va[m4] = tile + v_off + 32 * (m4 ^ ua);
    constexpr int kPv = DSA_MLA_PV_PREFETCH;
    bf16x8 vr[kPv];
    auto load_v = [&](int nb) {
      const int hi = 128 * (nb >> 2);
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(va[nb & 3] + hi));
      const bf16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(va[nb & 3] + 4 * kRowBytes + hi));
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int nb = 0; nb < kPv; ++nb) vr[nb] = load_v(nb);
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) {
      const bf16x8 vb = vr[nb % kPv];
      if (nb + kPv < 32) vr[nb % kPv] = load_v(nb + kPv);
      __builtin_amdgcn_sched_barrier(0);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pf, oacc[nb], 0, 0, 0);
    }
  };

  uint32_t slot_use = 0, slot_issue = kAhead * kTileBytes;   // byte offsets in the ring
  for (int it = 0; it < n_tiles; ++it) {
    // tiles it+1 .. it+kAhead-1 (those that exist) were issued after tile `it`
    const int younger = min(kAhead - 1, n_tiles - 1 - it);
    if (n_dma == 5) wait_younger<5>(younger);
    else wait_younger<4>(younger);
    // every wave's share of tile `it` has landed, and every wave is done with tile it-1
    // (whose slot the next load overwrites)
    lds_barrier();
    const uint8_t *tile = sh.tiles[0] + slot_use;
    if (mma) {
      f32x4 sc0, sc1;
      scores(tile, sc0, sc1);
      // the next tile's loads go out after the score product (measured faster than before
      // it: the score loads of every wave start right at the barrier)
      if (it + kAhead < n_tiles)
        issue_tile(sh.tiles[0] + slot_issue, sh.crow + (it + kAhead) * kTile, kv, td, n_dma, wave);
      accumulate(tile, weights(sc0, sc1, it));
    } else if (it + kAhead < n_tiles) {
      issue_tile(sh.tiles[0] + slot_issue, sh.crow + (it + kAhead) * kTile, kv, td, n_dma, wave);
    }
    // ring slots advance by one tile and wrap (uniform, loop-carried: no division)
    slot_use = slot_use + kTileBytes == kRing * kTileBytes ? 0u : slot_use + kTileBytes;
    slot_issue = slot_issue + kTileBytes == kRing * kTileBytes ? 0u : slot_issue + kTileBytes;
  }
  // every wave is done with the ring before it is reused for staging (no load is in flight:
  // the last iteration waited for all of them)
  lds_barrier();
  if (!mma) return;

  // ---- epilogue.  Lane (g, c) holds head h0 + c, dims 16nb + 4g + i.  The wave stages its
  // 16 x 512 block in LDS (the ring is free now) and writes it with 16-byte stores.  The
  // lane-derived addresses are recomputed from an opaque copy of the lane id: values kept
  // from the prologue would otherwise stay live across the whole loop.
  int le = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(le));
  const int ce = le & 15, ge = le >> 4;
  constexpr int kStageRow = kDv * 2 + 16;   // bytes per staged head row (padded)
  uint8_t *stage = sh.tiles[0] + wave * 16 * kStageRow;
  const float l_tot = sum_xor32(sum_xor16(l_part));
  const float linv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    const uint32_t lo = pack_bf16x2(oacc[nb][0] * linv, oacc[nb][1] * linv);
    const uint32_t hi = pack_bf16x2(oacc[nb][2] * linv, oacc[nb][3] * linv);
    *reinterpret_cast<uint2 *>(stage + ce * kStageRow + (16 * nb + 4 * ge) * 2) = make_uint2(lo, hi);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  uint16_t *dst;
  if (splits == 1) {
    dst = out + ((int64_t)r * H + h0) * kDv;
    if (lse && ge == 0) lse[(int64_t)r * H + h0 + ce] = lse2 * kLn2;
  } else {
    const int64_t ph0 = ((int64_t)r * splits + split) * H + h0;
    dst = part_o + ph0 * kDv;
    if (ge == 0) part_lse[ph0 + ce] = lse2;
  }
  // row j of the staged block = head h0 + j: 1024 bytes = 64 lanes x 16 B
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const i32x4 v = *reinterpret_cast<const i32x4 *>(stage + j * kStageRow + le * 16);
    *reinterpret_cast<i32x4 *>(dst + (int64_t)j * kDv + le * 8) = v;
  }
}

// Merge split partials: out = sum_s 2^(lse_s - lse) o_s with lse = log2 sum_s 2^lse_s.
// A workgroup merges kCombHeads heads of one row, one wave per head (thread: 8 dims of one
// head); workgroups are dealt to XCDs like the split workgroups of their row.
#ifndef DSA_COMB_HEADS
#define DSA_COMB_HEADS 4
#endif
constexpr int kCombHeads = DSA_COMB_HEADS;
constexpr int kCombThreads = kCombHeads * kWave;
constexpr int kMaxCombine = 32;   // largest split count
__global__ __launch_bounds__(kCombThreads) void mla_combine_kernel(int R, int H, int splits,
                                                          const uint16_t *__restrict__ part_o,
                                                          const float *__restrict__ part_lse,
                                                          uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per_row = H / kCombHeads;
  const int r = (j / per_row) * 8 + x;
  if (r >= R) return;
  const int h = (j % per_row) * kCombHeads + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  // every load is issued before any arithmetic (splits <= kMaxCombine)
  float ls[kMaxCombine];
  i32x4 pv[kMaxCombine];
#pragma unroll
  for (int s = 0; s < kMaxCombine; ++s) {
    if (s < splits) {
      const int64_t ph = ((int64_t)r * splits + s) * H + h;
      ls[s] = part_lse[ph];
      pv[s] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(part_o + ph * kDv + d0));
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxCombine; ++s)
    if (s < splits) m = fmaxf(m, ls[s]);
  float wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxCombine; ++s) {
      if (s < splits) {
        const float wgt = exp2f(ls[s] - m);
        wsum += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = (uint32_t)pv[s][e];
          acc[2 * e] = fmaf(wgt, bf16_bits_to_f32((uint16_t)(u & 0xFFFFu)), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wgt, bf16_bits_to_f32((uint16_t)(u >> 16)), acc[2 * e + 1]);
        }
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  i32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = (int)pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<i32x4 *>(out + ((int64_t)r * H + h) * kDv + d0) = o;
  if (lse && (threadIdx.x & 63) == 0)
    lse[(int64_t)r * H + h] = wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

#ifndef DSA_MLA_MIN_TILES
#define DSA_MLA_MIN_TILES 4
#endif
int mla_num_splits(int num_rows, int n_heads, int k) {
  // about one workgroup per CU for few-row batches, at least DSA_MLA_MIN_TILES tiles each
  const int base = num_rows * (n_heads / kHeadsPerBlock > 0 ? n_heads / kHeadsPerBlock : 1);
  int splits = (256 + base - 1) / base;
  const int max_splits = (k + DSA_MLA_MIN_TILES * kTile - 1) / (DSA_MLA_MIN_TILES * kTile);
  if (splits > max_splits) splits = max_splits;
  if (splits > kMaxCombine) splits = kMaxCombine;
  if (splits < 1) splits = 1;
  return splits;
}

size_t mla_workspace_bytes(int num_rows, int n_heads, int d_v, int k) {
  const int splits = mla_num_splits(num_rows, n_heads, k);
  if (splits <= 1) return 0;
  // bf16 partial outputs [R, splits, H, d_v], then fp32 partial log-sum-exps [R, splits, H]
  return (size_t)num_rows * splits * n_heads * (sizeof(uint16_t) * (size_t)d_v + sizeof(float));
}

template <bool PAGED, bool SEL, int HG>
static hipError_t launch_mla_kernel(unsigned grid, hipStream_t stream, const RowsDev &rows, int R,
                                    float sl2, const uint16_t *q16, const uint8_t *kv8,
                                    int32_t *idx, int k, int per, int splits, uint16_t *o16,
                                    float *lse, uint16_t *part_o, float *part_lse,
                                    const MlaSel &sel) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e =
      ensure_dynamic_lds(&mla_bf16_kernel<PAGED, SEL, HG>, (int)sizeof(MlaShared), lds_set);
  if (e != hipSuccess) return e;
  mla_bf16_kernel<PAGED, SEL, HG><<<grid, kMlaThreads, sizeof(MlaShared), stream>>>(
      R, splits, k, per, idx, q16, rows.row_seq, rows.row_len, rows.seq_start, rows.page_table,
      rows.max_pages, sl2, kv8, o16, lse, part_o, part_lse, sel);
  return hipGetLastError();
}

// idx is read (sel == nullptr) or written: with sel the kernel finishes the row's top-k from
// the chunked filter's survivors.
static hipError_t launch_bf16(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                              const void *kv, int32_t *idx, int k, void *out, float *lse,
                              int splits, void *ws, const MlaSel *sel, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  const int R = rh.num_rows;
  // A split batch small enough gives each (row, split) two workgroups of 64 heads.  A batch
  // of 8 or more splits per row that is too large for that trades half its splits for the two
  // head groups (half the partials to write and merge; measured faster at 32 rows of up to
  // 64K, the same at 64 rows of 8K with 4 splits, so batches of fewer splits keep them).
  int hg = (kMlaHeadGroups > 1 && splits > 1 && 8 * ((R + 7) / 8) * splits * 2 <= 256) ? 2 : 1;
  if (hg == 1 && kMlaHeadGroups > 1 && splits >= 8 &&
      8 * ((R + 7) / 8) * (splits / 2) * 2 <= 256) {
    splits /= 2;
    hg = 2;
  }
  const int per = (((k + splits - 1) / splits) + kTile - 1) / kTile * kTile;
  uint16_t *part_o = nullptr;
  float *part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<uint16_t *>(ws);
    part_lse = reinterpret_cast<float *>(part_o + (size_t)rh.num_rows * splits * H * kDv);
  }
  const unsigned grid = 8u * (unsigned)((R + 7) / 8) * splits * hg;
  const uint16_t *q16 = static_cast<const uint16_t *>(q);
  const uint8_t *kv8 = static_cast<const uint8_t *>(kv);
  uint16_t *o16 = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  const MlaSel none{};
  const MlaSel &sl = sel ? *sel : none;
  hipError_t e;
#define DSA_LAUNCH_MLA(P, S, G)                                                                 \
  launch_mla_kernel<P, S, G>(grid, stream, rows, R, sl2, q16, kv8, idx, k, per, splits, o16, lse, \
                             part_o, part_lse, sl)
  if (hg == 2)
    e = sel ? (paged ? DSA_LAUNCH_MLA(true, true, 2) : DSA_LAUNCH_MLA(false, true, 2))
            : (paged ? DSA_LAUNCH_MLA(true, false, 2) : DSA_LAUNCH_MLA(false, false, 2));
  else
    e = sel ? (paged ? DSA_LAUNCH_MLA(true, true, 1) : DSA_LAUNCH_MLA(false, true, 1))
            : (paged ? DSA_LAUNCH_MLA(true, false, 1) : DSA_LAUNCH_MLA(false, false, 1));
#undef DSA_LAUNCH_MLA
  if (e != hipSuccess || splits == 1) return e;
  mla_combine_kernel<<<8u * (unsigned)((R + 7) / 8) * (H / kCombHeads), kCombThreads, 0, stream>>>(
      R, H, splits, part_o, part_lse, o16, lse);
  return hipGetLastError();
}

hipError_t launch_mla_bf16(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                           const void *kv, const int32_t *idx, int k, void *out, float *lse,
                           int splits, void *ws, hipStream_t stream) {
  return launch_bf16(rh, paged, H, scale, q, kv, const_cast<int32_t *>(idx), k, out, lse, splits,
                     ws, nullptr, stream);
}

hipError_t launch_mla_bf16_select(const RowsHost &rh, bool paged, int H, float scale,
                                  const void *q, const void *kv, int32_t *idx, int k, void *out,
                                  float *lse, int splits, void *ws, const float *logits,
                                  int64_t ld, void *topk_ws, int hist_lists, hipStream_t stream) {
  MlaSel sel;
  sel.logits = logits;
  sel.ld = ld;
  sel.ws = topk_chunk_ws(topk_ws, rh.num_rows, rh.max_row_len, hist_lists);
  sel.chunks = (rh.max_row_len + kChunk - 1) / kChunk;
  return launch_bf16(rh, paged, H, scale, q, kv, idx, k, out, lse, splits, ws, &sel, stream);
}

}  // namespace dsa
