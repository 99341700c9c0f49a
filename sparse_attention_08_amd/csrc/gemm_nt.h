// gemm_nt.h -- C[m][n] = sum_k A[m][k] B[n][k] on gfx950 MFMA: bf16 operands whose
// contraction dimension is contiguous in memory (the rows of A and of B), fp32 accumulation,
// bf16 result.  The problem type supplies the addresses of the rows, so one kernel serves
// gathered rows (cache rows of a sequence's positions), per-head slices of a [R, H, D]
// tensor and plain matrices alike.
//
// A workgroup (4 waves) owns a 256 x 128 block of C (rows x columns).  The contraction runs
// in steps of 32: each thread fetches 16-byte pieces of the next step's A and B rows into
// registers while the waves multiply the current step out of LDS (two buffers, rows padded
// by 16 bytes so the operand reads of a 16-row block hit distinct banks).  Each wave holds a
// 128 x 64 block as 8 x 4 tiles of v_mfma_f32_16x16x32_bf16: per step 32 products for 12
// operand reads (a 64 x 64 block needs 8 reads for 16), two waves per SIMD.  The result is
// staged in LDS as bf16 and written back in 16-byte pieces, 256 bytes of a row per 16 lanes.
#pragma once
#include "dsa_device.h"

namespace dsa {

typedef int i32x2 __attribute__((ext_vector_type(2)));

struct GemmRow {
  const uint16_t *ptr;
  bool live;
};

constexpr int kGemmTile = 128;                      // columns of C per workgroup (N % 128 == 0)
constexpr int kGemmTileM = 256;                     // rows of C per workgroup
constexpr int kGemmK = 32;                          // contraction step
constexpr int kGemmThreads = 256;
constexpr int kGemmRow = kGemmK * 2 + 16;           // LDS bytes per operand row (padded)
constexpr int kGemmOpA = kGemmTileM * kGemmRow;     // one step of A: 20 KB
constexpr int kGemmOpB = kGemmTile * kGemmRow;      // one step of B: 10 KB
constexpr int kGemmOutRow = kGemmTile * 2 + 16;     // LDS bytes per staged result row
constexpr int kGemmLds = (2 * (kGemmOpA + kGemmOpB) > kGemmTileM * kGemmOutRow)
                             ? 2 * (kGemmOpA + kGemmOpB)
                             : kGemmTileM * kGemmOutRow;
constexpr int kGemmAPer = kGemmTileM * 4 / kGemmThreads;   // A pieces per thread and step: 4
constexpr int kGemmBPer = kGemmTile * 4 / kGemmThreads;    // B pieces: 2

// Prob: the problem, with (z = blockIdx.z, a batch index)
//   int M, N, K                        (N % 128 == 0, K % 32 == 0, K >= 32)
//   GemmRow a(int m, int z)            {row m of A (K contiguous, 16-byte aligned), live}: live
//                                      false when row m of C is not wanted (not computed, not
//                                      written; the pointer is then never read); called for
//                                      every m < M, best without branches, so that its loads
//                                      for a thread's rows go out together
//   const uint16_t *b(int n, int z)    row n of B (K contiguous, 16-byte aligned)
//   uint16_t *c(int m, int z)          row m of C (16-byte aligned); only called for live rows
// Grid: (N / 128, ceil(M / 256), batches).
template <class Prob>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_nt_kernel(Prob p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kGemmLds];
  __shared__ uint8_t live_row[kGemmTileM];
  auto opA = [&](int buf) { return lds + buf * kGemmOpA; };
  auto opB = [&](int buf) { return lds + 2 * kGemmOpA + buf * kGemmOpB; };
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // the wave's 128 x 64 block
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.y * kGemmTileM, n0 = blockIdx.x * kGemmTile, z = blockIdx.z;
  // thread t stages 16-byte piece (t & 3) of A rows (t >> 2) + 64 j and B rows (t >> 2) + 64 j
  const int lr = t >> 2, lc = t & 3;
  // A row that is not live reads a B row instead: its products only reach C rows that are not
  // written, and every load stays unconditional (no exec-masked branches in the loop, which
  // make the compiler wait for the A loads before it issues the B loads).
  const uint16_t *arow[kGemmAPer], *brow[kGemmBPer];
#pragma unroll
  for (int j = 0; j < kGemmBPer; ++j) brow[j] = p.b(n0 + lr + 64 * j, z) + 8 * lc;
  bool lv[kGemmAPer], any_live = false;
#pragma unroll
  for (int j = 0; j < kGemmAPer; ++j) {
    const int m = m0 + lr + 64 * j;
    const GemmRow a = p.a(m < p.M ? m : p.M - 1, z);
    lv[j] = m < p.M && a.live;
    any_live |= lv[j];
    arow[j] = lv[j] ? a.ptr + 8 * lc : brow[0];
  }
  if (lc == 0)
#pragma unroll
    for (int j = 0; j < kGemmAPer; ++j) live_row[lr + 64 * j] = lv[j];
  if (!__syncthreads_or(any_live)) return;   // nothing of this block is wanted
  i32x4 ra[kGemmAPer], rb[kGemmBPer];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kGemmAPer; ++j) ra[j] = *reinterpret_cast<const i32x4 *>(arow[j] + k0);
#pragma unroll
    for (int j = 0; j < kGemmBPer; ++j) rb[j] = *reinterpret_cast<const i32x4 *>(brow[j] + k0);
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kGemmAPer; ++j)
      *reinterpret_cast<i32x4 *>(opA(buf) + (lr + 64 * j) * kGemmRow + 16 * lc) = ra[j];
#pragma unroll
    for (int j = 0; j < kGemmBPer; ++j)
      *reinterpret_cast<i32x4 *>(opB(buf) + (lr + 64 * j) * kGemmRow + 16 * lc) = rb[j];
  };
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // operands: A rows 128 wm + 16 i + c and B rows 64 wn + 16 j + c, k = 8 g .. 8 g + 7
  auto products = [&](int buf) {
    bf16x8 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bv[j] = *reinterpret_cast<const bf16x8 *>(opB(buf) + (64 * wn + 16 * j + c) * kGemmRow + 16 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8 av =
          *reinterpret_cast<const bf16x8 *>(opA(buf) + (128 * wm + 16 * i + c) * kGemmRow + 16 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[j], av, acc[i][j], 0, 0, 0);
    }
  };
  fetch(0);
  stage(0);
  __syncthreads();
  // the last step is peeled off so that the loop body is one straight block
  const int steps = p.K / kGemmK;
  for (int s = 0; s + 1 < steps; ++s) {
    fetch((s + 1) * kGemmK);   // in flight during the products
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the products
    products(s & 1);
    __builtin_amdgcn_sched_barrier(0);   // and the stores (which wait for them) after
    stage((s & 1) ^ 1);        // that buffer's last readers passed the barrier below
    __syncthreads();
  }
  products((steps - 1) & 1);
  __syncthreads();             // the result staging below overwrites both buffers
  // result tile (i, j) (B is the products' first operand): lane (g, c) holds row
  // 128 wm + 16 i + c, columns 64 wn + 16 j + 4 g + q, q = 0..3 -- one 8-byte LDS write
  uint8_t *out = lds;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<i32x2 *>(out + (128 * wm + 16 * i + c) * kGemmOutRow +
                                 (64 * wn + 16 * j + 4 * g) * 2) =
          i32x2{(int)pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                (int)pack_bf16x2(acc[i][j][2], acc[i][j][3])};
  __syncthreads();
  // 16 threads per row, 16 bytes each
#pragma unroll
  for (int u = 0; u < kGemmTileM * kGemmTile / 8 / kGemmThreads; ++u) {
    const int id = u * kGemmThreads + t;
    const int row = id >> 4, piece = id & 15;
    const int m = m0 + row;
    if (live_row[row])
      *reinterpret_cast<i32x4 *>(p.c(m, z) + n0 + 8 * piece) =
          *reinterpret_cast<const i32x4 *>(out + row * kGemmOutRow + 16 * piece);
  }
}

}  // namespace dsa
