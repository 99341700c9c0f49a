// prep.hip -- indexer-input and cache-write prep on gfx950: the step in front of the
// lightning indexer on every new token ("DeepSeek-V3.2 技术报告摘要", section 1, DSA ①:
// indexer keys and queries, FP8 supported; "DeepSeek-V3.2-Exp" README, section "更新": the
// indexer's RoPE takes the non-interleaved layout, the MLA's RoPE the interleaved one;
// "DeepSeek-V3.2" model docs, section 5.3: bf16 latent cache in 64-token pages).
//
// RoPE of a 64-dim part x with the caller's table row cs = [cos_0..31 | sin_0..31]: pair i
// is (x[i], x[i+32]) in the non-interleaved layout and (x[2i], x[2i+1]) in the interleaved
// one, (a, b) -> (a cos_i - b sin_i, b cos_i + a sin_i).  Indexer vectors (128 dims) carry the
// rotation in dims 0..63, MLA vectors (576 dims) in dims 512..575.  fp8 quantisation of a
// 128-dim indexer vector y: scale = max|y| / 448 (1 for a zero vector), codes e4m3(y / scale)
// rounded to nearest even.  These end in rounding decisions, so every product, sum and
// quotient is one IEEE fp32 operation (no fused multiply-add) and the codes come from the
// hardware's round-to-nearest-even conversions.
//
// The work is a few KB per token and HBM-bound: one wave per token (key side) handles the
// 256-byte indexer key (a 32-bit pair of dims per lane, the rotation partner fetched with a
// lane exchange) and the 1152-byte latent entry (16 bytes per lane, the rotated tail as one
// pair per lane).
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kPrepWaves = 4;
constexpr int kPrepThreads = kPrepWaves * kWave;

__device__ __forceinline__ void rot_pair(float a, float b, float c, float s, float &ya, float &yb) {
#pragma clang fp contract(off)
  ya = a * c - b * s;
  yb = b * c + a * s;
}

// One wave: the 128-dim indexer vector whose dims 2l, 2l + 1 lane l loaded as `w` (bf16),
// rotated on dims 0..63 (non-interleaved), written to `out` as bf16 (dims 64..127 copied) or
// as e4m3 codes with *scale_out.  The rotation partner of lane l (dims 2l +- 32) is l ^ 16.
// The lane's angles (i = 2l mod 32 and i + 1, for lanes below 32), read once per position.
struct IdxAngles {
  float c0, c1, s0, s1;
};
__device__ __forceinline__ IdxAngles idx_angles(const float *cs, int lane) {
  const int i = (2 * lane) & 31;
  return {cs[i], cs[i + 1], cs[32 + i], cs[33 + i]};
}

template <bool FP8>
__device__ __forceinline__ void indexer_vec(uint32_t w, const IdxAngles &an, uint8_t *out,
                                            float *scale_out, int lane) {
  const uint32_t pw = (uint32_t)__shfl_xor((int)w, 16, kWave);
  float y0 = bf16_bits_to_f32(w & 0xffffu), y1 = bf16_bits_to_f32(w >> 16);
  if (lane < 32) {
    const float p0 = bf16_bits_to_f32(pw & 0xffffu), p1 = bf16_bits_to_f32(pw >> 16);
    const float c0 = an.c0, c1 = an.c1, s0 = an.s0, s1 = an.s1;
    float u0, u1, v0, v1;
    if (lane < 16) {   // first members of their pairs: a = own, b = partner
      rot_pair(y0, p0, c0, s0, u0, v0);
      rot_pair(y1, p1, c1, s1, u1, v1);
      y0 = u0;
      y1 = u1;
    } else {           // second members: a = partner, b = own
      rot_pair(p0, y0, c0, s0, u0, v0);
      rot_pair(p1, y1, c1, s1, u1, v1);
      y0 = v0;
      y1 = v1;
    }
  }
  if constexpr (!FP8) {
    reinterpret_cast<uint32_t *>(out)[lane] = lane < 32 ? pack_bf16x2(y0, y1) : w;
  } else {
    const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    const int code = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(y0, scale), __fdiv_rn(y1, scale), 0,
                                                     false);
    reinterpret_cast<uint16_t *>(out)[lane] = (uint16_t)(code & 0xffff);
    if (lane == 0) *scale_out = scale;
  }
}

// One wave: dims 512..575 of the 576-dim MLA vector `in` rotated (interleaved) into `out`;
// with COPY the latent dims 0..511 are copied too (16 bytes per lane).  `in` may be `out`.
template <bool COPY>
__device__ __forceinline__ void mla_vec(const uint16_t *in, const float *cs, uint16_t *out,
                                        int lane) {
  if constexpr (COPY)
    reinterpret_cast<i32x4 *>(out)[lane] = reinterpret_cast<const i32x4 *>(in)[lane];
  if (lane < 32) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(in + 512)[lane];
    float ya, yb;
    rot_pair(bf16_bits_to_f32(w & 0xffffu), bf16_bits_to_f32(w >> 16), cs[lane], cs[32 + lane], ya,
             yb);
    reinterpret_cast<uint32_t *>(out + 512)[lane] = pack_bf16x2(ya, yb);
  }
}

template <bool FP8>
__global__ __launch_bounds__(kPrepThreads) void prep_keys_kernel(
    int T, const int32_t *__restrict__ pos, const int64_t *__restrict__ rows, int64_t cache_rows,
    const float *__restrict__ cos_sin, int max_pos, const uint16_t *__restrict__ k_in,
    uint8_t *__restrict__ k_cache, float *__restrict__ k_scale, const uint16_t *__restrict__ kv_in,
    uint16_t *__restrict__ kv_cache) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kPrepWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int p = pos[t];
  const int64_t r = rows[t];
  if (p < 0 || p >= max_pos || r < 0 || r >= cache_rows) return;   // uniform per wave
  const float *cs = cos_sin + (int64_t)p * 64;
  const uint32_t w = reinterpret_cast<const uint32_t *>(k_in + (int64_t)t * 128)[lane];
  const IdxAngles an = idx_angles(cs, lane);
  mla_vec<true>(kv_in + (int64_t)t * 576, cs, kv_cache + r * 576, lane);
  indexer_vec<FP8>(w, an, k_cache + r * 128 * (FP8 ? 1 : 2), FP8 ? k_scale + r : nullptr, lane);
}

// Grid (rows, 4): part y of row r rotates indexer heads 16y .. 16y + 15 (4 per wave) and a
// quarter of the MLA heads (one pair per thread and step, in place).
template <bool FP8>
__global__ __launch_bounds__(kPrepThreads) void prep_queries_kernel(
    int R, const int32_t *__restrict__ pos, const float *__restrict__ cos_sin, int max_pos,
    const uint16_t *qi_in, uint8_t *qi_out, float *__restrict__ qi_scale, int n_heads,
    uint16_t *q) {
  const int r = blockIdx.x, part = blockIdx.y;
  const int p = pos[r];
  if (p < 0 || p >= max_pos) return;
  const float *cs = cos_sin + (int64_t)p * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every load of the workgroup's share is issued before the first store (the outputs may
  // alias the inputs, so the compiler would not hoist them itself)
  const int64_t v0 = (int64_t)r * 64 + 16 * part + 4 * wave;
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) w[hh] = reinterpret_cast<const uint32_t *>(qi_in + (v0 + hh) * 128)[lane];
  const int per_part = (n_heads + 3) / 4;
  const int h0 = part * per_part, h1 = min(n_heads, h0 + per_part);
  constexpr int kPairSteps = 4;   // pairs per thread held at once: 32 heads per part
  uint32_t *pr[kPairSteps];
  uint32_t pv[kPairSteps];
  const int i = threadIdx.x & 31;   // the angle is the same for every step of a thread
  const float c = cs[i], sn = cs[32 + i];
  const IdxAngles an = idx_angles(cs, lane);
  for (int j0 = 0; j0 < (h1 - h0) * 32; j0 += kPairSteps * kPrepThreads) {
#pragma unroll
    for (int u = 0; u < kPairSteps; ++u) {
      const int j = j0 + u * kPrepThreads + threadIdx.x;
      pr[u] = j < (h1 - h0) * 32
                  ? reinterpret_cast<uint32_t *>(q + ((int64_t)r * n_heads + h0 + (j >> 5)) * 576 + 512) + i
                  : nullptr;
      pv[u] = pr[u] ? *pr[u] : 0u;
    }
    if (j0 == 0) {
#pragma unroll
      for (int hh = 0; hh < 4; ++hh)
        indexer_vec<FP8>(w[hh], an, qi_out + (v0 + hh) * 128 * (FP8 ? 1 : 2),
                         FP8 ? qi_scale + v0 + hh : nullptr, lane);
    }
#pragma unroll
    for (int u = 0; u < kPairSteps; ++u) {
      if (!pr[u]) continue;
      float ya, yb;
      rot_pair(bf16_bits_to_f32(pv[u] & 0xffffu), bf16_bits_to_f32(pv[u] >> 16), c, sn, ya, yb);
      *pr[u] = pack_bf16x2(ya, yb);
    }
  }
  if (h1 <= h0) {   // no MLA heads in this part (fewer than 4 heads in all)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
      indexer_vec<FP8>(w[hh], an, qi_out + (v0 + hh) * 128 * (FP8 ? 1 : 2),
                       FP8 ? qi_scale + v0 + hh : nullptr, lane);
  }
}

hipError_t launch_prep_keys(int T, const int32_t *pos, const int64_t *rows, int64_t cache_rows,
                            const float *cos_sin, int max_pos, bool fp8, const void *k_in,
                            void *k_cache, float *k_scale, const void *kv_in, void *kv_cache,
                            hipStream_t stream) {
  const unsigned grid = (unsigned)((T + kPrepWaves - 1) / kPrepWaves);
  const uint16_t *ki = static_cast<const uint16_t *>(k_in);
  const uint16_t *kvi = static_cast<const uint16_t *>(kv_in);
  uint8_t *kc = static_cast<uint8_t *>(k_cache);
  uint16_t *kvc = static_cast<uint16_t *>(kv_cache);
  if (fp8)
    prep_keys_kernel<true><<<grid, kPrepThreads, 0, stream>>>(T, pos, rows, cache_rows, cos_sin,
                                                              max_pos, ki, kc, k_scale, kvi, kvc);
  else
    prep_keys_kernel<false><<<grid, kPrepThreads, 0, stream>>>(T, pos, rows, cache_rows, cos_sin,
                                                               max_pos, ki, kc, k_scale, kvi, kvc);
  return hipGetLastError();
}

hipError_t launch_prep_queries(int R, const int32_t *pos, const float *cos_sin, int max_pos,
                               bool fp8, const void *qi_in, void *qi_out, float *qi_scale,
                               int n_heads, void *q, hipStream_t stream) {
  const dim3 grid((unsigned)R, 4);
  const uint16_t *qi = static_cast<const uint16_t *>(qi_in);
  uint8_t *qo = static_cast<uint8_t *>(qi_out);
  uint16_t *qq = static_cast<uint16_t *>(q);
  if (fp8)
    prep_queries_kernel<true><<<grid, kPrepThreads, 0, stream>>>(R, pos, cos_sin, max_pos, qi, qo,
                                                                 qi_scale, n_heads, qq);
  else
    prep_queries_kernel<false><<<grid, kPrepThreads, 0, stream>>>(R, pos, cos_sin, max_pos, qi, qo,
                                                                  qi_scale, n_heads, qq);
  return hipGetLastError();
}

}  // namespace dsa
