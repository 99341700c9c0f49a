// dsa_device.h -- device-side helpers shared by the DSA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kPage = 64;          // tokens per cache page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Where query rows find their cache: contiguous (seq_start) or 64-token pages.
// Grids with one row per block index: the y dimension of a grid holds at most 65535 blocks,
// so rows beyond it continue in z (grid (x, min(R, 65535), ceil(R / 65535)), launched by
// row_grid); blocks past the last row return at once.
__device__ __forceinline__ int grid_row() { return (int)(blockIdx.y + gridDim.y * blockIdx.z); }

struct RowsDev {
  const int32_t *row_seq;
  const int32_t *row_len;
  const int64_t *seq_start;   // contiguous layout, else nullptr
  const int32_t *page_table;  // paged layout, else nullptr
  int32_t max_pages;
};

template <bool PAGED>
__device__ __forceinline__ int64_t cache_row(const RowsDev &rows, int b, int64_t s) {
  if constexpr (PAGED) {
    int64_t page = rows.page_table[(int64_t)b * rows.max_pages + (s >> 6)];
    return page * kPage + (s & (kPage - 1));
  } else {
    return rows.seq_start[b] + s;
  }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> packed bf16 pair (a in the low half), round to nearest even in hardware.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Weighted sum over the 64 indexer heads of a 16-key score tile, on the matrix cores.
// The tile's scores are the four 16x16 head blocks of an MFMA result: lane (g, c) holds
// S[16 hb + 4g + i][key c] in acc[hb][i].  Two head blocks at a time, ReLU'd and rounded to
// bf16, form the B operand (K = 32 heads) of a 16x16x32 bf16 MFMA whose A operand holds the
// matching head weights in every row; each output row is then sum_h w[h] relu(S[h][c]), so
// every lane (g, c) receives the score of key c, accumulated in fp32.  Lane group g's K
// slots hold its own heads 16 hb + 4g + i in both operands, so the weights of a lane are
// the ones it already holds.  Against an fp32 epilogue this rounds each weighted term's
// two factors to bf16 (relative 2^-9 each) and replaces 32 VALU operations per tile by
// 16 and two MFMAs.
typedef short i16x2 __attribute__((ext_vector_type(2)));
struct HeadWeights {
  bf16x8 a[2];   // A operands: heads of blocks {0, 1} and {2, 3}
};
// ReLU of two floats as a packed bf16 pair: one conversion and a packed signed 16-bit max
// on the bits (negative values and -0 compare below 0).
__device__ __forceinline__ uint32_t relu_bf16x2(float a, float b) {
  i16x2 v = __builtin_bit_cast(i16x2, __builtin_convertvector((f32x2{a, b}), bf16x2));
  v = __builtin_elementwise_max(v, (i16x2){0, 0});
  return __builtin_bit_cast(uint32_t, v);
}
// wt[hb][i]: the weight of head 16 hb + 4g + i (g = lane / 16); element j of a[p] is head
// block 2p + j / 4, row j % 4
__device__ __forceinline__ HeadWeights head_weights(const float (&wt)[4][4]) {
  HeadWeights hw;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const i32x4 v = {(int)pack_bf16x2(wt[2 * p][0], wt[2 * p][1]),
                     (int)pack_bf16x2(wt[2 * p][2], wt[2 * p][3]),
                     (int)pack_bf16x2(wt[2 * p + 1][0], wt[2 * p + 1][1]),
                     (int)pack_bf16x2(wt[2 * p + 1][2], wt[2 * p + 1][3])};
    hw.a[p] = __builtin_bit_cast(bf16x8, v);
  }
  return hw;
}
__device__ __forceinline__ float head_sum(const f32x4 (&acc)[4], const HeadWeights &hw) {
  f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const i32x4 b = {(int)relu_bf16x2(acc[2 * p][0], acc[2 * p][1]),
                     (int)relu_bf16x2(acc[2 * p][2], acc[2 * p][3]),
                     (int)relu_bf16x2(acc[2 * p + 1][0], acc[2 * p + 1][1]),
                     (int)relu_bf16x2(acc[2 * p + 1][2], acc[2 * p + 1][3])};
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hw.a[p], __builtin_bit_cast(bf16x8, b), d, 0, 0, 0);
  }
  return d[0];
}

// Leading radix digit of the top-k select: sign, exponent and 3 mantissa bits of the key.
constexpr int kLeadDigitBits = 12;
constexpr int kLeadBins = 1 << kLeadDigitBits;

// Order-preserving map of a finite float to uint32 (larger float -> larger key),
// with -0 folded onto +0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every vector
// memory operation of the wave (vmcnt(0)), which would drain global->LDS loads that are
// meant to stay in flight across the barrier; here only LDS operations (lgkmcnt) are
// completed first.  The signal fences keep the compiler from moving memory accesses
// across it.  Global->LDS loads a wave issued must be awaited with its own vmcnt wait.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// max(x, 0) as a signed-integer max on the bits: negative floats (and -0) have the sign
// bit set and compare below 0, so this is ReLU in one instruction (no NaN quieting).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Butterfly partners across lane rows with gfx950's VALU lane swaps (no LDS round trip):
// the value of lane l ^ 16, and of lane l ^ 32.  Called with both operands equal, the
// swap leaves lane l's own value in one half of the result and the partner's in the
// other, always in (lower lane, upper lane) order.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4 and 8
// lanes inside each row of 16 (lanes shifted in from outside the row add 0), then row 0's
// total is added to row 1 and row 2's to row 3 (broadcast of lane 15 of each row), then
// the running total at lane 31 is added to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2, 3
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

}  // namespace dsa
