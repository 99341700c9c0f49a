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
constexpr int kMlaWaves = 8;                 // 4 head groups x 2 value halves
constexpr int kMlaThreads = kMlaWaves * kWave;
constexpr int kHeadsPerBlock = 64;
constexpr int kRing = DSA_MLA_DEPTH;          // LDS tile slots (kRing - 1 tiles in flight)
constexpr int kMaxSlotsPerSplit = 2048;
static_assert(kTileBytes % 1024 == 0, "tile DMA is whole 1 KB instructions");

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
  uint32_t crow[kMaxSlotsPerSplit];        // cache row of each slot of the split
  uint32_t valid[kMaxSlotsPerSplit / 32];  // one bit per slot
  float xmax[4][2][16];                    // per head group, half: tile max of each head
  uint2 xp[4][2][kWave];                   // per head group, half: 4 bf16 weights per lane
  float xl[4][2][16];                      // final partial sums of the two halves
};

// The 36 DMA instructions of a tile go to waves 0..7 in turn (waves 0-3 issue 5, 4-7
// issue 4).  LDS position P = 1024*j + 16*lane of the tile holds entry P / 1152,
// physical chunk (P % 1152) / 16, i.e. logical chunk physical ^ swz(entry).
constexpr int kTileDma = kTileBytes / 1024;   // 36
__device__ __forceinline__ int tile_dma_count(int wave) {
  return kTileDma / kMlaWaves + (wave < kTileDma % kMlaWaves ? 1 : 0);
}
__device__ __forceinline__ void issue_tile(uint8_t *dst, const uint32_t *crow_tile,
                                          const uint8_t *__restrict__ kv, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < (kTileDma + kMlaWaves - 1) / kMlaWaves; ++i) {
    const int j = wave + kMlaWaves * i;
    if (j < kTileDma) {
      const int pos = 1024 * j + 16 * lane;
      const int e = pos / kRowBytes;
      const int pch = (pos - e * kRowBytes) >> 4;
      const int lch = pch ^ swz(e);
      const uint8_t *src = kv + (int64_t)crow_tile[e] * kRowBytes + 16 * lch;
      __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(dst + 1024 * j), 16, 0, 0);
    }
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

// Wave (hg, half) owns heads h0..h0+15 (hg = wave % 4) and value dims [256*half, +256)
// (half = wave / 4).  Per tile it scores entries 8g + 4*half + i (i < 4) of its lane
// row g: one 16-row MFMA block of S^T = C . Q^T.  The pair of waves sharing hg trade
// their per-head tile maxima and their bf16 weights through LDS, so each then holds the
// weights of all 32 entries for O^T += V^T . P^T over its value half.
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
  const int hg = wave & 3, half = wave >> 2;
  const int c = lane & 15, g = lane >> 4;
  const int len = rows.row_len[r], b = rows.row_seq[r];
  const int h0 = co.hgrp * kHeadsPerBlock + hg * 16;
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

  f32x4 oacc[16];
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // prologue: tiles 0 .. kRing-2 in flight (past the end: re-read the last tile, harmless)
  if (n_tiles > 0) {
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d) {
      const int t = min(d, n_tiles - 1);
      issue_tile(sh.tiles[d], sh.crow + t * kTile, kv, wave, lane);
    }
  }
  // rows of the score tile this lane feeds as the MFMA A operand: result rows 4g+i map
  // to entries 8g + 4*half + i
  const int arow = 8 * (c >> 2) + (c & 3) + 4 * half;
  const int a_even = 16 * (g ^ swz(arow)), a_odd = 16 * ((4 + g) ^ swz(arow));
  const int tr_i = c >> 2, tr_q = c & 3;
  const int swa = swz(8 * g + tr_i), swb = swz(8 * g + tr_i + 4);
  int offa[4], offb[4];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    offa[m4] = 16 * ((2 * m4 + (tr_q >> 1)) ^ swa);
    offb[m4] = 16 * ((2 * m4 + (tr_q >> 1)) ^ swb);
  }
  const int n_dma = tile_dma_count(wave);

  for (int it = 0; it < n_tiles; ++it) {
    // the slot of tile it-1 is free once every wave has passed the previous iteration
    __syncthreads();
    {
      const int t = min(it + kRing - 1, n_tiles - 1);
      issue_tile(sh.tiles[(it + kRing - 1) % kRing], sh.crow + t * kTile, kv, wave, lane);
    }
    if (n_dma == 5) __builtin_amdgcn_s_waitcnt(vmcnt_only(5 * (kRing - 1)));
    else __builtin_amdgcn_s_waitcnt(vmcnt_only(4 * (kRing - 1)));
    __syncthreads();   // every wave's share of tile `it` has landed
    const uint32_t valid = sh.valid[it];
    if (valid == 0) continue;
    const uint8_t *tile = sh.tiles[it % kRing];
    // ---- scores of entries 8g + 4*half + i for head c, K = 576 in 18 steps of 32
    const uint8_t *ab = tile + arow * kRowBytes;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};   // even / odd k-steps
#pragma unroll
    for (int t = 0; t < 18; t += 2) {
      const bf16x8 x0 = *reinterpret_cast<const bf16x8 *>(ab + 128 * (t >> 1) + a_even);
      const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(ab + 128 * (t >> 1) + a_odd);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, qf[t], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, qf[t + 1], s1, 0, 0, 0);
    }
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      z[i] = ((valid >> (8 * g + 4 * half + i)) & 1u) ? (s0[i] + s1[i]) * scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mx = max_xor32(max_xor16(mx));   // this half's maximum for head c
    if (g == 0) sh.xmax[hg][half][c] = mx;
    __syncthreads();
    mx = fmaxf(mx, sh.xmax[hg][half ^ 1][c]);   // finite: the tile has a valid entry
    // ---- lazy online softmax (log2 domain): the reference maximum only moves when the
    // tile maximum exceeds it by more than 8, so weights stay <= 2^8 and the rescale of
    // the accumulators is rare.  Both waves of the pair take identical decisions.
    const bool first = m_run == -INFINITY;
    const bool move = first || mx > m_run + 8.f;
    if (__ballot(move && !first)) {
      const float alpha = move ? exp2f(m_run - mx) : 1.f;
#pragma unroll
      for (int nb = 0; nb < 16; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] *= alpha;
      l_run *= alpha;
    }
    if (move) m_run = mx;
    float p[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(z[i] - m_run);
      ps += p[i];
    }
    l_run += sum_xor32(sum_xor16(ps));   // this half's entries only
    const uint32_t plo = (uint32_t)f32_to_bf16_bits(p[0]) | ((uint32_t)f32_to_bf16_bits(p[1]) << 16);
    const uint32_t phi = (uint32_t)f32_to_bf16_bits(p[2]) | ((uint32_t)f32_to_bf16_bits(p[3]) << 16);
    sh.xp[hg][half][lane] = make_uint2(plo, phi);
    __syncthreads();
    const uint2 oth = sh.xp[hg][half ^ 1][lane];
    // B operand P^T: entries 8g + e (e < 4 from half 0, e >= 4 from half 1), head c
    const uint2 p_lo = half == 0 ? make_uint2(plo, phi) : oth;
    const uint2 p_hi = half == 0 ? oth : make_uint2(plo, phi);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(p_lo.x, p_lo.y, p_hi.x, p_hi.y));
    // ---- O^T += V^T . P^T over this wave's value half: dv rows 256*half + 16nb + c
    const uint8_t *vab = tile + (8 * g + tr_i) * kRowBytes + 8 * (tr_q & 1) + 512 * half;
    const uint8_t *vbb = vab + 4 * kRowBytes;
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      const int hi = 128 * (nb >> 2);
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_ptr)(vab + hi + offa[nb & 3]));
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (lds_bf16x4_ptr)(vbb + hi + offb[nb & 3]));
      const bf16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pf, oacc[nb], 0, 0, 0);
    }
  }

  // no LDS write may still be in flight when the workgroup's LDS is reused or released
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  // the two halves' sums make the full softmax denominator
  if (g == 0) sh.xl[hg][half][c] = l_run;
  __syncthreads();
  const float l_tot = sh.xl[hg][0][c] + sh.xl[hg][1][c];
  const float linv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
  // ---- epilogue.  Lane (g, c) holds head h0 + c, dims 256*half + 16nb + 4g + i.  The
  // wave stages its 16 x 256 bf16 block in LDS (the tile ring is free now) and writes it
  // back with 16-byte stores.
  constexpr int kStageRow = 256 * 2 + 16;   // bytes per staged head row (padded)
  uint8_t *stage = sh.tiles[0] + wave * 16 * kStageRow;
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) {
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
    dst = out + ((int64_t)r * H + h0) * kDv + 256 * half;
    if (lse && g == 0 && half == 0) lse[(int64_t)r * H + h0 + c] = lse2 * kLn2;
  } else {
    const int64_t ph0 = ((int64_t)r * splits + split) * H + h0;
    dst = part_o + ph0 * kDv + 256 * half;
    if (g == 0 && half == 0) part_lse[ph0 + c] = lse2;
  }
  // row j of the staged block = head h0 + j: 512 bytes = 32 lanes x 16 B; two rows per store
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const int row = j + (lane >> 5), col = lane & 31;
    const i32x4 v = *reinterpret_cast<const i32x4 *>(stage + row * kStageRow + col * 16);
    *reinterpret_cast<i32x4 *>(dst + (int64_t)row * kDv + col * 8) = v;
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
