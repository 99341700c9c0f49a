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
//   int M, N, K                        (N % 128 == 0, K % 32 == 0)
//   bool live(int m, int z)            row m of C is computed and written
//   const uint16_t *a(int m, int z)    row m of A (K contiguous, 16-byte aligned); only
//                                      called for live rows
//   const uint16_t *b(int n, int z)    row n of B (K contiguous, 16-byte aligned)
//   uint16_t *c(int m, int z)          row m of C (16-byte aligned); only called for live rows
// Grid: (N / 128, ceil(M / 256), batches).
template <class Prob>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_nt_kernel(Prob p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kGemmLds];
  auto opA = [&](int buf) { return lds + buf * kGemmOpA; };
  auto opB = [&](int buf) { return lds + 2 * kGemmOpA + buf * kGemmOpB; };
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // the wave's 128 x 64 block
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.y * kGemmTileM, n0 = blockIdx.x * kGemmTile, z = blockIdx.z;
  // thread t stages 16-byte piece (t & 3) of A rows (t >> 2) + 64 j and B rows (t >> 2) + 64 j
  const int lr = t >> 2, lc = t & 3;
  const uint16_t *arow[kGemmAPer], *brow[kGemmBPer];
  bool any_live = false;
#pragma unroll
  for (int j = 0; j < kGemmAPer; ++j) {
    const int m = m0 + lr + 64 * j;
    const bool lv = m < p.M && p.live(m, z);
    any_live |= lv;
    arow[j] = lv ? p.a(m, z) + 8 * lc : nullptr;
  }
#pragma unroll
  for (int j = 0; j < kGemmBPer; ++j) brow[j] = p.b(n0 + lr + 64 * j, z) + 8 * lc;
  if (!__syncthreads_or(any_live)) return;   // nothing of this block is wanted
  i32x4 ra[kGemmAPer], rb[kGemmBPer];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kGemmAPer; ++j)
      ra[j] = arow[j] ? *reinterpret_cast<const i32x4 *>(arow[j] + k0) : i32x4{0, 0, 0, 0};
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
  fetch(0);
  stage(0);
  __syncthreads();
  const int steps = p.K / kGemmK;
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    if (s + 1 < steps) fetch((s + 1) * kGemmK);   // in flight during the products
    // operands: A rows 128 wm + 16 i + c and B rows 64 wn + 16 j + c, k = 8 g .. 8 g + 7
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
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < steps) stage(buf ^ 1);   // that buffer's last readers passed the barrier below
    __syncthreads();
  }
  // result tile (i, j): lane (g, c) holds rows 128 wm + 16 i + 4 g + q, column 64 wn + 16 j + c
  uint8_t *out = lds;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint16_t *>(out + (128 * wm + 16 * i + 4 * g + q) * kGemmOutRow +
                                      (64 * wn + 16 * j + c) * 2) = f32_to_bf16_bits(acc[i][j][q]);
  __syncthreads();
  // 16 threads per row, 16 bytes each
#pragma unroll
  for (int u = 0; u < kGemmTileM * kGemmTile / 8 / kGemmThreads; ++u) {
    const int id = u * kGemmThreads + t;
    const int row = id >> 4, piece = id & 15;
    const int m = m0 + row;
    if (m < p.M && p.live(m, z))
      *reinterpret_cast<i32x4 *>(p.c(m, z) + n0 + 8 * piece) =
          *reinterpret_cast<const i32x4 *>(out + row * kGemmOutRow + 16 * piece);
  }
}

}  // namespace dsa
