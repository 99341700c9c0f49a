// mha.hip -- masked MHA mode for short prefill on gfx950 ("DeepSeek-V3.2 技术报告摘要",
// section 1, "短序列优化": for short prefill DSA is run as masked MHA; "DeepSeek-V3.2 -- Model
// techniques map", "Multi-head latent attention": per head 128 nope + 64 rope query/key dims
// and 128 value dims, decompressed from the 512-dim latent).
//
// Step 1 decompresses the latent entries the batch can reach: for each sequence b, its
// positions s below the longest row_len of its rows (its reach), K_nope[b, s, h] = W_UK[h] c
// and V[b, s, h] = W_UV[h] c of the latent c at the cache row of (b, s), 128 dims each, bf16,
// into a compact [B, max_row_len, H, 128] layout (a gather GEMM, gemm_nt.h); cache rows no
// sequence reaches are never read.  Step 2 attends: row r, head h, over its sequence's
// positions s (all s < row_len, or the set of its top-k entries):
// z_s = scale [q_nope | q_rope] . [K_nope[s, h] | kr_s], out = softmax(z) V, lse = ln sum e^z.
//
// Attention kernel: a workgroup owns 128 consecutive query rows (4 waves x 2 blocks of 16) of
// one head.  Key tiles of 32 positions (K_nope 8 KB + RoPE keys 4 KB + V 8 KB) go through a
// 3-stage LDS ring (two tiles in flight) with global->LDS loads, each 1 KB instruction filled
// by one wave.  Each wave computes the transposed score tiles S^T = K . Q^T (keys as MFMA
// rows, its rows as columns, q in registers, each key operand load serving both row blocks),
// an online softmax in the log2 domain, and O^T += V^T . P^T
// with V^T read through the transposing LDS read; key rows of the score blocks are permuted
// (block kb, row 4g + i <-> key 8g + 4kb + i) so each lane's weights are the B operand of
// the value product as they stand.  Rows of one workgroup that belong to different
// sequences are handled one sequence at a time.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "gemm_nt.h"

namespace dsa {

constexpr int kMhaWaves = 4;
constexpr int kMhaThreads = kMhaWaves * kWave;
constexpr int kRowBlocks = 2;                  // 16-row blocks per wave
constexpr int kMhaRows = 16 * kRowBlocks * kMhaWaves;   // query rows per workgroup
constexpr int kMhaRing = 3;                    // LDS stages (two tiles in flight)
constexpr int kMhaKeys = 32;                   // keys per tile
constexpr int kNopeBytes = kMhaKeys * 256;     // 32 x 128 dims bf16
constexpr int kRopeBytes = kMhaKeys * 128;     // 32 x 64 dims bf16
constexpr int kValBytes = kMhaKeys * 256;      // 32 x 128 dims bf16
constexpr int kMaskOff = kNopeBytes + kRopeBytes + kValBytes;     // masked mode: the rows'
constexpr int kMhaStage = kMaskOff + 4 * 128;  // mask words of the tile (4 B per row)
constexpr int kMhaDma = kMaskOff / 1024;       // 20 key / value instructions of 1 KB
static_assert(kMhaDma % kMhaWaves == 0, "the DMA instructions split evenly over the waves");
constexpr int kMhaDmaPerWave = kMhaDma / kMhaWaves;   // 5
constexpr int kMhaMaxPages = 256;              // pages of one sequence held in LDS (16K tokens)

// Chunk swizzles (16-byte chunk x of key row j sits at x ^ swz(j)): the score operand reads
// (16 permuted key rows, one chunk per lane group) then touch 32 distinct 16-byte slots per
// half-wave, the condition measured for conflict-free ds_read_b128 on gfx950.
__device__ __forceinline__ int nope_swz(int j) { return (j & 3) | ((j >> 1) & 12); }
__device__ __forceinline__ int rope_swz(int j) { return ((j >> 3) & 3) << 1; }
// Value rows: the 32-byte column pair a transposing read takes from 8 rows (keys 8g + 0..3 for
// two lane groups) lands in 8 distinct 32-byte bank windows.
__device__ __forceinline__ int val_swz(int j) { return ((j & 3) | (((j >> 3) & 1) << 2)) << 1; }

__device__ __forceinline__ void mha_dma4(const void *src, const void *lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(la)
                   : "memory");
}
__device__ __forceinline__ void mha_dma16(const void *src, const void *lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(la)
                   : "memory");
}

typedef bf16x4 __attribute__((address_space(3))) *mha_lds_bf16x4_ptr;

// s_waitcnt with vmcnt <= n, other counters unconstrained (gfx9 field layout).
constexpr int mha_vmcnt(int n) { return (n & 0xF) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8); }

struct MhaShared {
  uint8_t stage[kMhaRing][kMhaStage];
  int32_t pages[kMhaMaxPages];
  int32_t seq[kMhaRows];
  int32_t len[kMhaRows];
};

// Two waves per SIMD (two workgroups per CU): up to 256 registers per lane for the two row
// blocks' queries and accumulators.
template <bool PAGED, bool MASKED>
__global__ __launch_bounds__(kMhaThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
mha_prefill_kernel(
    int R, int H, int n_row_tiles, const int32_t *__restrict__ row_seq,
    const int32_t *__restrict__ row_len, const int64_t *__restrict__ seq_start,
    const int32_t *__restrict__ page_table, int max_pages, float scale_log2,
    const uint16_t *__restrict__ q, const uint8_t *__restrict__ k_nope,
    const uint8_t *__restrict__ vals, const uint8_t *__restrict__ kv,
    const uint32_t *__restrict__ mask, int mask_words, uint16_t *__restrict__ out,
    float *__restrict__ lse, int lmax) {
  __shared__ __attribute__((aligned(16))) MhaShared sh;
  // longest row tiles (most keys) first; the heads of one row tile are consecutive workgroups
  const int rt = n_row_tiles - 1 - (int)(blockIdx.x / H);
  const int h = blockIdx.x % H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int r0 = rt * kMhaRows;
  if (threadIdx.x < kMhaRows) {
    const int rr = r0 + threadIdx.x;
    sh.seq[threadIdx.x] = rr < R ? row_seq[rr] : -1;
    sh.len[threadIdx.x] = rr < R ? row_len[rr] : 0;
  }
  // the wave's row blocks: rows r0 + 32 wave + 16 rb + c (column c of block rb's tiles);
  // q^T operand of block rb: dims 32t + 8g .. + 8 (t < 4: nope, t = 4, 5: rope)
  int my_r[kRowBlocks];
  bf16x8 qf[kRowBlocks][6];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    my_r[rb] = r0 + 32 * wave + 16 * rb + c;
    const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
        q + ((int64_t)(my_r[rb] < R ? my_r[rb] : 0) * H + h) * 192 + 8 * g);
#pragma unroll
    for (int t = 0; t < 6; ++t) qf[rb][t] = qp[4 * t];
  }
  __syncthreads();
  int my_seq[kRowBlocks], my_len[kRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    my_seq[rb] = sh.seq[32 * wave + 16 * rb + c];
    my_len[rb] = sh.len[32 * wave + 16 * rb + c];
  }

  f32x4 oacc[kRowBlocks][8];
  float m_run[kRowBlocks], l_part[kRowBlocks];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) oacc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_part[rb] = 0.f;
  }

  // score operand rows: block kb, lane row c <-> key 8 (c >> 2) + (c & 3) + 4 kb; lane group g
  // reads logical chunk 4t + g (nope: t < 4, 256-byte rows) or 4(t - 4) + g (rope, 128-byte
  // rows), stored at chunk ^ swz(key).  One operand load serves both row blocks.
  const int arow0 = 8 * (c >> 2) + (c & 3);
  int a_nope[2], a_rope[2], s_nope[2], s_rope[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int a = arow0 + 4 * kb;
    a_nope[kb] = a * 256;
    s_nope[kb] = nope_swz(a);
    a_rope[kb] = kNopeBytes + a * 128;
    s_rope[kb] = rope_swz(a);
  }
  // value operand: transposing reads of keys 8g + (c >> 2) (and + 4: same swizzle), dims
  // 16 nb + 4 (c & 3): logical chunk 2 nb + ((c & 3) >> 1) at chunk ^ val_swz(key)
  const int vrow = 8 * g + (c >> 2);
  const int v_off = kNopeBytes + kRopeBytes + vrow * 256 + 8 * (c & 3);
  const int v_sw = val_swz(vrow) >> 1;
  // LDS addresses of every operand read in ring slot 0 (a tile in slot i reads them plus
  // i * kMhaStage: one add per read).  Opaque to the compiler, which would otherwise fold the
  // shared block's address back in and spend two adds per read.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)sh.stage[0];
  uint32_t qk_addr[6][2], pv_addr[8];
#pragma unroll
  for (int t = 0; t < 6; ++t)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      qk_addr[t][kb] = lds0 + (t < 4 ? a_nope[kb] + 16 * ((4 * t + g) ^ s_nope[kb])
                                     : a_rope[kb] + 16 * ((4 * (t - 4) + g) ^ s_rope[kb]));
      __asm__ volatile("" : "+v"(qk_addr[t][kb]));
    }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    pv_addr[nb] = lds0 + v_off + 32 * (nb ^ v_sw);
    __asm__ volatile("" : "+v"(pv_addr[nb]));
  }
  // this wave's DMA instructions: i = wave + 4 u (u < 5); 0..7 nope (4 keys each), 8..11 rope
  // (8 keys each), 12..19 values (4 keys each)
  int d_key[kMhaDmaPerWave], d_src[kMhaDmaPerWave];
#pragma unroll
  for (int u = 0; u < kMhaDmaPerWave; ++u) {
    const int i = wave + kMhaWaves * u;
    if (i < 8) {
      d_key[u] = 4 * i + (lane >> 4);
      d_src[u] = 16 * ((lane & 15) ^ nope_swz(d_key[u]));
    } else if (i < 12) {
      d_key[u] = 8 * (i - 8) + (lane >> 3);
      d_src[u] = 16 * ((lane & 7) ^ rope_swz(d_key[u]));
    } else {
      d_key[u] = 4 * (i - 12) + (lane >> 4);
      d_src[u] = 16 * ((lane & 15) ^ val_swz(d_key[u]));
    }
  }

  uint64_t done[kMhaRows / 64] = {};
  for (;;) {
    // the next sequence among the workgroup's rows and its longest row
    int b = -1, kmax = 0;
    for (int i = 0; i < kMhaRows; ++i) {
      const int sq = sh.seq[i];
      if (sq < 0 || ((done[i >> 6] >> (i & 63)) & 1ull)) continue;
      if (b < 0) b = sq;
      if (sq == b) {
        kmax = max(kmax, sh.len[i]);
        done[i >> 6] |= 1ull << (i & 63);
      }
    }
    if (b < 0) break;
    bool mine[kRowBlocks];
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) mine[rb] = my_seq[rb] == b;
    const int n_tiles = (kmax + kMhaKeys - 1) / kMhaKeys;
    int64_t base = 0;
    // every wave is done with the previous sequence's tiles (the ring is reused from slot 0)
    // and page list
    __syncthreads();
    if constexpr (PAGED) {
      const int n_pages = (kmax + 63) / 64;
      for (int i = threadIdx.x; i < n_pages; i += kMhaThreads)
        sh.pages[i] = page_table[(int64_t)b * max_pages + i];
      __syncthreads();
    } else {
      base = seq_start[b];
    }
    auto cache_row = [&](int s) -> int64_t {
      if constexpr (PAGED)
        return (int64_t)sh.pages[s >> 6] * 64 + (s & 63);
      else
        return base + s;
    };
    // per-lane source bases of the wave's instructions (per tile, the key's row is added: its
    // compact row b * lmax + s for the decompressed keys and values, its cache row for the
    // RoPE keys, which come from the latent cache)
    const int64_t cbase = (int64_t)b * lmax;
    const uint8_t *src_base[kMhaDmaPerWave];
    int64_t src_stride[kMhaDmaPerWave];
    bool dec[kMhaDmaPerWave];
#pragma unroll
    for (int u = 0; u < kMhaDmaPerWave; ++u) {
      const int i = wave + kMhaWaves * u;
      dec[u] = i < 8 || i >= 12;
      if (i < 8) {
        src_base[u] = k_nope + (int64_t)h * 256 + d_src[u];
        src_stride[u] = (int64_t)H * 256;
      } else if (i < 12) {
        src_base[u] = kv + 1024 + d_src[u];
        src_stride[u] = 1152;
      } else {
        src_base[u] = vals + (int64_t)h * 256 + d_src[u];
        src_stride[u] = (int64_t)H * 256;
      }
    }
    // per-lane source of each DMA instruction at key d_key[u] of a tile whose first key is
    // cache row 0: a full tile adds its first key's cache row times the stride (uniform)
    const uint8_t *lane_src[kMhaDmaPerWave];
#pragma unroll
    for (int u = 0; u < kMhaDmaPerWave; ++u)
      lane_src[u] = src_base[u] + (int64_t)d_key[u] * src_stride[u];
    auto issue = [&](int tile, uint8_t *st) {
      if constexpr (MASKED)
        if (wave < kMhaRows / 64) {   // rows 64 wave .. + 63: their mask word of this tile
          const int rr = min(r0 + 64 * wave + lane, R - 1);
          mha_dma4(mask + (int64_t)rr * mask_words + tile, st + kMaskOff + 256 * wave);
        }
      if ((tile + 1) * kMhaKeys <= kmax) {
        // every key of the tile exists: 32 consecutive cache rows (half of one page when paged)
        // and 32 consecutive compact rows
        int64_t row0;
        if constexpr (PAGED)
          row0 = (int64_t)__builtin_amdgcn_readfirstlane(sh.pages[tile >> 1]) * 64 +
                 (tile & 1) * kMhaKeys;
        else
          row0 = base + (int64_t)tile * kMhaKeys;
        const int64_t crow0 = cbase + (int64_t)tile * kMhaKeys;
#pragma unroll
        for (int u = 0; u < kMhaDmaPerWave; ++u)
          mha_dma16(lane_src[u] + (dec[u] ? crow0 : row0) * src_stride[u],
                    st + 1024 * (wave + kMhaWaves * u));
      } else {
#pragma unroll
        for (int u = 0; u < kMhaDmaPerWave; ++u) {
          const int s = min(tile * kMhaKeys + d_key[u], kmax - 1);   // tail keys re-read the last
          mha_dma16(lane_src[u] + ((dec[u] ? cbase + s : cache_row(s)) - d_key[u]) * src_stride[u],
                    st + 1024 * (wave + kMhaWaves * u));
        }
      }
    };
    for (int t0 = 0; t0 < kMhaRing - 1 && t0 < n_tiles; ++t0) issue(t0, sh.stage[t0]);
    // loads per tile issued by this wave (the only vector-memory operations of the loop)
    const int n_dma = kMhaDmaPerWave + ((MASKED && wave < kMhaRows / 64) ? 1 : 0);
    // one tile in ring slot `slot`
    auto step = [&](int j, int slot) {
      // this wave's part of tile j has landed once at most the younger tiles' loads are in
      // flight; every wave is done with tile j - 1, whose slot the next load reuses
      if (min(kMhaRing - 2, n_tiles - 1 - j) >= 1) {
        if (n_dma == kMhaDmaPerWave) __builtin_amdgcn_s_waitcnt(mha_vmcnt(kMhaDmaPerWave));
        else __builtin_amdgcn_s_waitcnt(mha_vmcnt(kMhaDmaPerWave + 1));
      } else {
        __builtin_amdgcn_s_waitcnt(mha_vmcnt(0));
      }
      lds_barrier();
      if (j + kMhaRing - 1 < n_tiles)
        issue(j + kMhaRing - 1, sh.stage[slot == 0 ? kMhaRing - 1 : slot - 1]);
      const uint8_t *st = sh.stage[slot];
      const uint32_t slot_off = (uint32_t)slot * kMhaStage;
      uint32_t mword[kRowBlocks] = {};
      if constexpr (MASKED)
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
          mword[rb] = reinterpret_cast<const uint32_t *>(st + kMaskOff)[32 * wave + 16 * rb + c];
      // ---- S^T for the tile's 32 keys (2 blocks of 16) x the wave's 2 x 16 rows
      f32x4 sc[kRowBlocks][2];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb)
        sc[rb][0] = sc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 6; ++t) {
        bf16x8 x[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          x[kb] = *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)(qk_addr[t][kb] +
                                                                                 slot_off);
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            sc[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[kb], qf[rb][t], sc[rb][kb],
                                                                 0, 0, 0);
      }
      // ---- per row block: mask (key s = 32 j + 8g + 4 kb + i attended by the row iff the
      // row belongs to this sequence, s < len, and, masked, bit s of its mask is set) and the
      // online softmax in the log2 domain (the reference maximum moves only when the tile
      // maximum exceeds it by more than 8: weights stay <= 2^8, rescales are rare)
      bf16x8 pf[kRowBlocks];
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        // raw scores; masked entries -inf (the scale is applied in the exponent, scale > 0)
        float p[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[4 * kb + i] = sc[rb][kb][i];
        // dense mode: a tile below every row's length needs no mask (all but the last tiles)
        const bool full = !MASKED && __all(mine[rb] && (j + 1) * kMhaKeys <= my_len[rb]);
        if (!full) {
          const int s0 = j * kMhaKeys + 8 * g;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // non-short-circuit tests and a select: one compare chain and a v_cndmask per
              // score (short-circuit forms were compiled to a branch per score)
              bool ok = mine[rb] & ((s0 + 4 * kb + i) < my_len[rb]);
              if constexpr (MASKED) ok = ok & (((mword[rb] >> (8 * g + 4 * kb + i)) & 1u) != 0u);
              p[4 * kb + i] = ok ? p[4 * kb + i] : -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])),
                         fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7])));
        mx = max_xor32(max_xor16(mx)) * scale_log2;
        const bool move = mx > -INFINITY && (m_run[rb] == -INFINITY || mx > m_run[rb] + 8.f);
        if (__ballot(move && m_run[rb] > -INFINITY)) {
          const float alpha =
              (move && m_run[rb] > -INFINITY) ? __builtin_amdgcn_exp2f(m_run[rb] - mx) : 1.f;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[rb][nb][i] *= alpha;
          l_part[rb] *= alpha;
        }
        if (move) m_run[rb] = mx;
        const float neg_m = m_run[rb] > -INFINITY ? -m_run[rb] : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(p[i], scale_log2, neg_m));
        l_part[rb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pf[rb] = __builtin_bit_cast(
            bf16x8, make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                               pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
      }
      // ---- O^T += V^T . P^T, value rows 16 nb + c; one operand load serves both row blocks
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint32_t va = pv_addr[nb] + slot_off;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((mha_lds_bf16x4_ptr)(uintptr_t)va);
        const bf16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((mha_lds_bf16x4_ptr)(uintptr_t)(va + 4 * 256));
        const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rb = 0; rb < kRowBlocks; ++rb)
          oacc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rb], oacc[rb][nb], 0, 0, 0);
      }
    };
    for (int j = 0, slot = 0; j < n_tiles; ++j, slot = slot == kMhaRing - 1 ? 0 : slot + 1)
      step(j, slot);
  }

  // ---- epilogue: lane (g, c) holds row my_r[rb], value dims 16 nb + 4g + i
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb) {
    const float l = sum_xor32(sum_xor16(l_part[rb]));
    if (my_r[rb] >= R) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t *o = out + ((int64_t)my_r[rb] * H + h) * 128 + 4 * g;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint2 v = make_uint2(pack_bf16x2(oacc[rb][nb][0] * inv, oacc[rb][nb][1] * inv),
                                 pack_bf16x2(oacc[rb][nb][2] * inv, oacc[rb][nb][3] * inv));
      *reinterpret_cast<uint2 *>(o + 16 * nb) = v;
    }
    if (lse && g == 0)
      lse[(int64_t)my_r[rb] * H + h] = l > 0.f ? (m_run[rb] + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// Mask bits of the top-k sets: word w of row r holds positions 32 w .. 32 w + 31.
__global__ __launch_bounds__(256) void mha_mask_clear_kernel(uint32_t *__restrict__ mask,
                                                             int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    mask[i] = 0u;
}
__global__ __launch_bounds__(256) void mha_mask_set_kernel(const int32_t *__restrict__ idx, int k,
                                                           const int32_t *__restrict__ row_len,
                                                           uint32_t *__restrict__ mask,
                                                           int mask_words) {
  const int r = blockIdx.x;
  const int len = row_len[r];
  for (int j = threadIdx.x; j < k; j += 256) {
    const int s = idx[(int64_t)r * k + j];
    if (s >= 0 && s < len) atomicOr(&mask[(int64_t)r * mask_words + (s >> 5)], 1u << (s & 31));
  }
}

// Reach of each sequence: the longest row_len among its rows (0 without rows).
__global__ __launch_bounds__(256) void mha_reach_kernel(const int32_t *__restrict__ row_seq,
                                                        const int32_t *__restrict__ row_len, int R,
                                                        int32_t *__restrict__ reach) {
  __shared__ int32_t wmax[256 / kWave];
  const int b = blockIdx.x;
  int m = 0;
  for (int r = threadIdx.x; r < R; r += 256)
    if (row_seq[r] == b) m = max(m, row_len[r]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 256 / kWave; ++w) m = max(m, wmax[w]);
    reach[b] = max(m, wmax[0]);
  }
}

// The decompression as a gather GEMM: C row m = compact row (b = m / lmax, s = m % lmax),
// live while s < reach[b]; its A row is the latent c (first 512 of 576) at the cache row of
// (b, s); B row n = row n of W_UK (z = 0) or W_UV (z = 1) viewed as [H * 128, 512]; C row m
// of K_nope (z = 0) or V (z = 1), [B * lmax, H * 128].  The lookups are unconditional (b < B
// and s >> 6 < max_pages for every m < M), so a thread's rows load them together.
template <bool PAGED>
struct MhaDecompress {
  int M, N, K;
  const uint16_t *kv;
  const int64_t *seq_start;
  const int32_t *page_table;
  int max_pages, lmax;
  const int32_t *reach;
  const uint16_t *w[2];
  uint16_t *dst[2];
  __device__ GemmRow a(int m, int) const {
    const int b = m / lmax, s = m - b * lmax;
    int64_t row;
    if constexpr (PAGED)
      row = (int64_t)page_table[(int64_t)b * max_pages + (s >> 6)] * 64 + (s & 63);
    else
      row = seq_start[b] + s;
    // the live test reads the row lookup too (a cache row is never negative), so neither
    // load can be moved under the test: a thread's lookups go out together, not one by one
    return {kv + row * 576, (s < reach[b]) && (row >= 0)};
  }
  __device__ const uint16_t *b(int n, int z) const { return w[z] + (int64_t)n * 512; }
  __device__ uint16_t *c(int m, int z) const { return dst[z] + (int64_t)m * N; }
};

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// [B] reaches, then K_nope and V ([B, max_row_len, H, 128] bf16 each), then the masks
size_t mha_workspace_bytes(int num_seqs, int H, int R, int max_row_len, bool masked) {
  const size_t dec = (size_t)num_seqs * max_row_len * H * 128 * 2;
  const size_t m = masked ? (size_t)R * ((max_row_len + 31) / 32) * 4 : 0;
  return a256(4 * (size_t)num_seqs) + 2 * a256(dec) + m;
}

hipError_t launch_mha_prefill(const RowsHost &rh, bool paged, int H, float scale, const void *q,
                              const void *kv, const void *w_uk, const void *w_uv,
                              const int32_t *idx, int k, void *out, float *lse, void *ws,
                              hipStream_t stream) {
  const int B = rh.num_seqs, L = rh.max_row_len;
  const size_t dec_bytes = a256((size_t)B * L * H * 128 * 2), reach_bytes = a256(4 * (size_t)B);
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  int32_t *reach = reinterpret_cast<int32_t *>(wsb);
  uint16_t *k_nope = reinterpret_cast<uint16_t *>(wsb + reach_bytes);
  uint16_t *vals = reinterpret_cast<uint16_t *>(wsb + reach_bytes + dec_bytes);
  uint32_t *mask =
      idx ? reinterpret_cast<uint32_t *>(wsb + reach_bytes + 2 * dec_bytes) : nullptr;
  const int mask_words = (L + 31) / 32;
  mha_reach_kernel<<<B, 256, 0, stream>>>(rh.row_seq, rh.row_len, rh.num_rows, reach);
  const dim3 dgrid((unsigned)H, (unsigned)(((int64_t)B * L + kGemmTileM - 1) / kGemmTileM), 2);
  const auto *kv16 = static_cast<const uint16_t *>(kv);
  const auto *wk = static_cast<const uint16_t *>(w_uk);
  const auto *wv = static_cast<const uint16_t *>(w_uv);
  if (paged) {
    const MhaDecompress<true> pr{B * L, H * 128, 512, kv16, rh.seq_start, rh.page_table,
                                 rh.max_pages, L, reach, {wk, wv}, {k_nope, vals}};
    gemm_nt_kernel<<<dgrid, kGemmThreads, 0, stream>>>(pr);
  } else {
    const MhaDecompress<false> pr{B * L, H * 128, 512, kv16, rh.seq_start, rh.page_table,
                                  rh.max_pages, L, reach, {wk, wv}, {k_nope, vals}};
    gemm_nt_kernel<<<dgrid, kGemmThreads, 0, stream>>>(pr);
  }
  if (idx) {
    const int64_t n = (int64_t)rh.num_rows * mask_words;
    mha_mask_clear_kernel<<<(unsigned)std::min<int64_t>((n + 255) / 256, 4096), 256, 0, stream>>>(
        mask, n);
    mha_mask_set_kernel<<<rh.num_rows, 256, 0, stream>>>(idx, k, rh.row_len, mask, mask_words);
  }
  const int n_row_tiles = (rh.num_rows + kMhaRows - 1) / kMhaRows;
  const unsigned grid = (unsigned)n_row_tiles * (unsigned)H;
  const float scale_log2 = scale * kLog2e;
  const auto *qq = static_cast<const uint16_t *>(q);
  const auto *kn = reinterpret_cast<const uint8_t *>(k_nope);
  const auto *vv = reinterpret_cast<const uint8_t *>(vals);
  const auto *kvb = static_cast<const uint8_t *>(kv);
  auto *oo = static_cast<uint16_t *>(out);
#define DSA_MHA_ARGS                                                                           \
  rh.num_rows, H, n_row_tiles, rh.row_seq, rh.row_len, rh.seq_start, rh.page_table,          \
      rh.max_pages, scale_log2, qq, kn, vv, kvb, mask, mask_words, oo, lse, L
  if (paged) {
    if (idx) mha_prefill_kernel<true, true><<<grid, kMhaThreads, 0, stream>>>(DSA_MHA_ARGS);
    else mha_prefill_kernel<true, false><<<grid, kMhaThreads, 0, stream>>>(DSA_MHA_ARGS);
  } else {
    if (idx) mha_prefill_kernel<false, true><<<grid, kMhaThreads, 0, stream>>>(DSA_MHA_ARGS);
    else mha_prefill_kernel<false, false><<<grid, kMhaThreads, 0, stream>>>(DSA_MHA_ARGS);
  }
#undef DSA_MHA_ARGS
  return hipGetLastError();
}

}  // namespace dsa
