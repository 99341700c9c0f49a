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
// bf16 kernel design.  A workgroup owns one query row, 64 heads (4 waves x 16 heads)
// and a range of top-k slots.  The cache rows of all its slots are resolved up front;
// selected entries are then gathered 32 at a time from HBM straight into a ring of LDS
// tiles with direct global->LDS loads (several tiles in flight, no staging registers),
// the XOR swizzle applied through the choice of source chunk.  Each wave computes the transposed
// score tile S^T = C . Q^T (keys as MFMA rows, its 16 heads as columns, q resident in
// registers), runs the online softmax in fp32 in the log2 domain, and accumulates
// O += P . V with V read from the same LDS tile through the gfx950 transposing LDS
// read (ds_read_b64_tr_b16), so the tile is stored once, row-major, for both products.
// The LDS tile uses an XOR swizzle of 16-byte chunks so that both the row reads of the
// score product and the transposed reads of the value product are conflict-free.
// Few-row (decode) batches split the slots over several workgroups; each writes a
// normalised bf16 partial and its log-sum-exp, and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

// ------------------------------------------------------------------------------------
// fp32 path: one workgroup per (row, head), two passes over the selected entries.
// ------------------------------------------------------------------------------------
template <bool PAGED>
__global__ __launch_bounds__(256) void mla_f32_kernel(RowsDev rows, int H, int Dqk, int Dv,
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
  const int h = blockIdx.x, r = blockIdx.y;
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
  dim3 grid(H, rh.num_rows);
  const size_t shm = sizeof(float) * ((k + 1) & ~1) + sizeof(int64_t) * k + sizeof(float) * Dqk;
  if (paged)
    mla_f32_kernel<true><<<grid, 256, shm, stream>>>(rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                     lse);
  else
    mla_f32_kernel<false><<<grid, 256, shm, stream>>>(rows, H, Dqk, Dv, scale, q, kv, idx, k, out,
                                                      lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// bf16 MFMA path, d_qk = 576 (512 latent + 64 RoPE), d_v = 512.
// ------------------------------------------------------------------------------------
#ifndef DSA_MLA_DEPTH
#define DSA_MLA_DEPTH 4
#endif
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;          // 1152 B per cache entry
constexpr int kTile = 32;                    // entries per LDS tile
constexpr int kTileBytes = kTile * kRowBytes;   // 36 KB = 36 DMA instructions of 1 KB
constexpr int kMlaThreads = 256;             // 4 waves x 16 heads
constexpr int kMlaWaves = kMlaThreads / kWave;
constexpr int kHeadsPerBlock = 64;
constexpr int kRing = DSA_MLA_DEPTH;          // LDS tile slots (kRing - 1 tiles in flight)
constexpr int kMaxSlotsPerSplit = 2048;
constexpr int kDmaPerWave = kTileBytes / 1024 / kMlaWaves;   // 9
static_assert(kTileBytes % (1024 * kMlaWaves) == 0, "tile DMA must split evenly over waves");

// XOR swizzle of the 16-byte chunk index inside its aligned group of 8 chunks.
__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 3) & 1); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

typedef bf16x4 __attribute__((address_space(3))) *lds_bf16x4_ptr;
typedef void __attribute__((address_space(3))) *lds_void_ptr;

constexpr int vmcnt_only(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

struct MlaShared {
  uint8_t tiles[kRing][kTileBytes];
  uint32_t crow[kMaxSlotsPerSplit];      // cache row of each slot of the split
  uint32_t valid[kMaxSlotsPerSplit / 32];  // one bit per slot
};

// This wave's share of the DMA of tile `t` into `dst`: LDS position P = 1024*j + 16*lane of
// the tile holds entry P / 1152, physical chunk (P % 1152) / 16, i.e. logical chunk
// physical ^ swz(entry) of that entry's cache row.
__device__ __forceinline__ void issue_tile(uint8_t *dst, const uint32_t *crow_tile,
                                          const uint8_t *__restrict__ kv, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int j = wave * kDmaPerWave + i;
    const int pos = 1024 * j + 16 * lane;
    const int e = pos / kRowBytes;
    const int pch = (pos - e * kRowBytes) >> 4;
    const int lch = pch ^ swz(e);
    const uint8_t *src = kv + (int64_t)crow_tile[e] * kRowBytes + 16 * lch;
    __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(dst + 1024 * j), 16, 0, 0);
  }
}

// Workgroup -> (row, head group, split).  Workgroups are dealt to the 8 XCDs round-robin by
// id, so all workgroups of a row (its splits and both head groups) land on one XCD: the
// gathered entries are shared through that XCD's L2 and the partials stay in it.
struct MlaCoord { int r, hgrp, split; };
__device__ __forceinline__ bool mla_coord(int bid, int R, int HG, int S, MlaCoord &c) {
  const int x = bid & 7, j = bid >> 3;
  c.r = (j / (HG * S)) * 8 + x;
  const int rem = j % (HG * S);
  c.hgrp = rem / S;
  c.split = rem % S;
  return c.r < R;
}

template <bool PAGED>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    RowsDev rows, int R, int H, float scale_log2, const uint16_t *__restrict__ q,
    const uint8_t *__restrict__ kv, const int32_t *__restrict__ idx, int k, int slots_per_split,
    int splits, uint16_t *__restrict__ out, float *__restrict__ lse, uint16_t *__restrict__ part_o,
    float *__restrict__ part_lse) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_smem[];
  MlaShared &sh = *reinterpret_cast<MlaShared *>(mla_smem);
  MlaCoord co;
  if (!mla_coord(blockIdx.x, R, H / kHeadsPerBlock, splits, co)) return;
  const int r = co.r, split = co.split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r], b = rows.row_seq[r];
  const int h0 = co.hgrp * kHeadsPerBlock + wave * 16;
  const int slot_begin = split * slots_per_split;
  const int slot_end = min(k, slot_begin + slots_per_split);
  const int n_slots = max(0, slot_end - slot_begin);
  const int n_tiles = (n_slots + kTile - 1) / kTile;
  const int32_t *idx_row = idx + (int64_t)r * k;

  // q^T operand: head h0 + c, dims 32t + 8g .. +8 for t < 18 (in flight during the
  // slot resolution below)
  bf16x8 qf[18];
  {
    const bf16x8 *qp =
        reinterpret_cast<const bf16x8 *>(q + ((int64_t)r * H + h0 + c) * kDqk + 8 * g);
#pragma unroll
    for (int t = 0; t < 18; ++t) qf[t] = qp[4 * t];
  }
  // cache rows and validity of every slot of the split (invalid slots read position 0)
  const int64_t row_of_0 = cache_row<PAGED>(rows, b, 0);
  for (int t0 = 0; t0 < n_tiles * kTile; t0 += kMlaThreads) {
    const int t = t0 + threadIdx.x;
    int s = -1;
    if (t < n_slots) s = idx_row[slot_begin + t];
    const bool ok = t < n_slots && s >= 0 && s < len;
    const uint64_t vm = __ballot(ok);
    if (t < n_tiles * kTile) sh.crow[t] = (uint32_t)(ok ? cache_row<PAGED>(rows, b, s) : row_of_0);
    if (lane == 0 && t < n_tiles * kTile) sh.valid[t >> 5] = (uint32_t)vm;
    if (lane == 32 && t < n_tiles * kTile) sh.valid[t >> 5] = (uint32_t)(vm >> 32);
  }
  __syncthreads();

  f32x4 oacc[32];
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // prologue: tiles 0 .. kRing-2 in flight (past the end: re-read the last tile, harmless)
  if (n_tiles > 0) {
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d) {
      const int t = min(d, n_tiles - 1);
      issue_tile(sh.tiles[d], sh.crow + t * kTile, kv, wave, lane);
    }
  }
  const int arow0 = 8 * (c >> 2) + (c & 3);
  const int arow1 = arow0 + 4;
  const int tr_i = c >> 2, tr_q = c & 3;

  for (int it = 0; it < n_tiles; ++it) {
    // the slot of tile it-1 is free once every wave has passed the previous iteration
    __syncthreads();
    {
      const int t = min(it + kRing - 1, n_tiles - 1);
      issue_tile(sh.tiles[(it + kRing - 1) % kRing], sh.crow + t * kTile, kv, wave, lane);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(kDmaPerWave * (kRing - 1)));
    __syncthreads();   // every wave's share of tile `it` has landed
    const uint32_t valid = sh.valid[it];
    if (valid == 0) continue;
    const uint8_t *tile = sh.tiles[it % kRing];
    // ---- scores S^T (entries x heads), K = 576 in 18 steps of 32.  Chunk 4t + g of row
    // arow sits at 128*(t/2) + 16*(((4*(t&1)) + g) ^ swz(arow)): two per-lane bases plus
    // compile-time offsets.
    const uint8_t *a0b = tile + arow0 * kRowBytes;
    const uint8_t *a1b = tile + arow1 * kRowBytes;
    const int a0e = 16 * (g ^ swz(arow0)), a0o = 16 * ((4 + g) ^ swz(arow0));
    const int a1e = 16 * (g ^ swz(arow1)), a1o = 16 * ((4 + g) ^ swz(arow1));
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 18; ++t) {
      const int hi = 128 * (t >> 1);
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(a0b + hi + ((t & 1) ? a0o : a0e));
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(a1b + hi + ((t & 1) ? a1o : a1e));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[t], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[t], s1, 0, 0, 0);
    }
    // ---- online softmax for head c over entries 8g .. 8g+7 (log2 domain).  The reference
    // maximum m_run is only moved when the tile maximum exceeds it by more than 8 (a factor
    // 256): weights then stay <= 2^8, fp32 accumulation is unaffected, and the rescale of
    // the 128 accumulator registers is rare instead of per tile.
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ((valid >> (8 * g + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
      z[4 + i] = ((valid >> (8 * g + 4 + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
    mx = max_xor32(max_xor16(mx));                  // finite: the tile has a valid entry
    const bool first = m_run == -INFINITY;          // accumulators still zero
    const bool move = first || mx > m_run + 8.f;
    if (__ballot(move && !first)) {
      const float alpha = move ? exp2f(m_run - mx) : 1.f;
#pragma unroll
      for (int nb = 0; nb < 32; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] *= alpha;
      l_run *= alpha;
    }
    if (move) m_run = mx;
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(z[e] - m_run);
      ps += p[e];
    }
    l_run += sum_xor32(sum_xor16(ps));
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (__bf16)p[e];
    // ---- O^T += V^T . P^T: A = V^T (dv rows 16nb + c, entries 8g + e via two transposing
    // LDS reads), B = P^T (entries 8g + e, head c); result rows dv 16nb + 4g + i, column
    // head c.  Chunk 2nb + (tr_q >> 1) of row ra sits at 128*(nb/4) + one of 4 per-lane
    // offsets (nb % 4).
    const uint8_t *vab = tile + (8 * g + tr_i) * kRowBytes + 8 * (tr_q & 1);
    const uint8_t *vbb = vab + 4 * kRowBytes;
    const int swa = swz(8 * g + tr_i), swb = swz(8 * g + tr_i + 4);
    int offa[4], offb[4];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) {
      offa[m4] = 16 * ((2 * m4 + (tr_q >> 1)) ^ swa);
      offb[m4] = 16 * ((2 * m4 + (tr_q >> 1)) ^ swb);
    }
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) {
      const int hi = 128 * (nb >> 2);
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_ptr)(vab + hi + offa[nb & 3]));
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_ptr)(vbb + hi + offb[nb & 3]));
      const bf16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pf, oacc[nb], 0, 0, 0);
    }
  }

  // no LDS write may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  // ---- epilogue.  Lane (g, c) holds head h0 + c, dims 16nb + 4g + i.  The wave stages
  // its 16 x 512 bf16 block in LDS (the tile ring is free now) and writes it back with
  // 16-byte stores, 1 KB (one head row) per instruction.
  const float linv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse2 = l_run > 0.f ? m_run + log2f(l_run) : -INFINITY;
  __syncthreads();
  constexpr int kStageRow = kDv * 2 + 16;   // bytes per staged head row (padded)
  uint8_t *stage = sh.tiles[0] + wave * 16 * kStageRow;
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) {
    const uint32_t lo = (uint32_t)f32_to_bf16_bits(oacc[nb][0] * linv) |
                        ((uint32_t)f32_to_bf16_bits(oacc[nb][1] * linv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_bits(oacc[nb][2] * linv) |
                        ((uint32_t)f32_to_bf16_bits(oacc[nb][3] * linv) << 16);
    *reinterpret_cast<uint2 *>(stage + c * kStageRow + (16 * nb + 4 * g) * 2) = make_uint2(lo, hi);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  uint16_t *dst;
  if (splits == 1) {
    dst = out + ((int64_t)r * H + h0) * kDv;
    if (lse && g == 0) lse[(int64_t)r * H + h0 + c] = lse2 * kLn2;
  } else {
    const int64_t ph0 = ((int64_t)r * splits + split) * H + h0;
    dst = part_o + ph0 * kDv;
    if (g == 0) part_lse[ph0 + c] = lse2;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const i32x4 v = *reinterpret_cast<const i32x4 *>(stage + j * kStageRow + lane * 16);
    *reinterpret_cast<i32x4 *>(dst + (int64_t)j * kDv + lane * 8) = v;
  }
}

// Merge split partials: out = sum_s 2^(lse_s - lse) o_s with lse = log2 sum_s 2^lse_s.
// A workgroup of 256 threads merges 4 heads of one row (thread: 8 dims of one head);
// workgroups are dealt to XCDs like the split workgroups of their row.
constexpr int kCombHeads = 4;
constexpr int kMaxCombine = 16;   // largest split count
__global__ __launch_bounds__(256) void mla_combine_kernel(int R, int H, int splits,
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
    o[e] = (int)((uint32_t)f32_to_bf16_bits(acc[2 * e] * inv) |
                 ((uint32_t)f32_to_bf16_bits(acc[2 * e + 1] * inv) << 16));
  *reinterpret_cast<i32x4 *>(out + ((int64_t)r * H + h) * kDv + d0) = o;
  if (lse && (threadIdx.x & 63) == 0)
    lse[(int64_t)r * H + h] = wsum > 0.f ? (m + log2f(wsum)) * kLn2 : -INFINITY;
}

int mla_num_splits(int num_rows, int n_heads, int k) {
  const int base = num_rows * (n_heads / kHeadsPerBlock > 0 ? n_heads / kHeadsPerBlock : 1);
  int splits = (256 + base - 1) / base;
  const int max_splits = (k + 4 * kTile - 1) / (4 * kTile);   // at least 4 tiles per split
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

template <bool PAGED>
static hipError_t launch_mla_kernel(unsigned grid, hipStream_t stream, const RowsDev &rows, int R,
                                    int H, float sl2, const uint16_t *q16, const uint8_t *kv8,
                                    const int32_t *idx, int k, int per, int splits, uint16_t *o16,
                                    float *lse, uint16_t *part_o, float *part_lse) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mla_bf16_kernel<PAGED>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(MlaShared));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  mla_bf16_kernel<PAGED><<<grid, kMlaThreads, sizeof(MlaShared), stream>>>(
      rows, R, H, sl2, q16, kv8, idx, k, per, splits, o16, lse, part_o, part_lse);
  return hipGetLastError();
}

hipError_t launch_mla_bf16(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                           const void *kv, const int32_t *idx, int k, void *out, float *lse,
                           int splits, void *ws, hipStream_t stream) {
  RowsDev rows{rh.row_seq, rh.row_len, rh.seq_start, rh.page_table, rh.max_pages};
  const int per = (((k + splits - 1) / splits) + kTile - 1) / kTile * kTile;
  uint16_t *part_o = nullptr;
  float *part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<uint16_t *>(ws);
    part_lse = reinterpret_cast<float *>(part_o + (size_t)rh.num_rows * splits * H * kDv);
  }
  const int R = rh.num_rows, HG = H / kHeadsPerBlock;
  const unsigned grid = 8u * (unsigned)((R + 7) / 8) * HG * splits;
  const uint16_t *q16 = static_cast<const uint16_t *>(q);
  const uint8_t *kv8 = static_cast<const uint8_t *>(kv);
  uint16_t *o16 = static_cast<uint16_t *>(out);
  const float sl2 = scale * kLog2e;
  hipError_t e = paged ? launch_mla_kernel<true>(grid, stream, rows, R, H, sl2, q16, kv8, idx, k,
                                                 per, splits, o16, lse, part_o, part_lse)
                       : launch_mla_kernel<false>(grid, stream, rows, R, H, sl2, q16, kv8, idx, k,
                                                  per, splits, o16, lse, part_o, part_lse);
  if (e != hipSuccess || splits == 1) return e;
  mla_combine_kernel<<<8u * (unsigned)((R + 7) / 8) * (H / kCombHeads), 256, 0, stream>>>(
      R, H, splits, part_o, part_lse, o16, lse);
  return hipGetLastError();
}

}  // namespace dsa
