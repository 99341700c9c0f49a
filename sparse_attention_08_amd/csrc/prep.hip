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

// Key side, one wave per token t: every input load (the token's position and cache row, its
// indexer key and latent entry) is issued before the position is checked.
template <bool FP8>
__device__ __forceinline__ void prep_key_wave(int t, const int32_t *__restrict__ pos,
                                              const int64_t *__restrict__ rows, int64_t cache_rows,
                                              const float *__restrict__ cos_sin, int max_pos,
                                              const uint16_t *__restrict__ k_in,
                                              uint8_t *__restrict__ k_cache,
                                              float *__restrict__ k_scale,
                                              const uint16_t *__restrict__ kv_in,
                                              uint16_t *__restrict__ kv_cache, int lane) {
  const int p = pos[t];
  const int64_t r = rows[t];
  const uint32_t w = reinterpret_cast<const uint32_t *>(k_in + (int64_t)t * 128)[lane];
  const uint16_t *kvt = kv_in + (int64_t)t * 576;
  const i32x4 latent = reinterpret_cast<const i32x4 *>(kvt)[lane];
  const uint32_t tail = lane < 32 ? reinterpret_cast<const uint32_t *>(kvt + 512)[lane] : 0u;
  if (p < 0 || p >= max_pos || r < 0 || r >= cache_rows) return;   // uniform per wave
  const float *cs = cos_sin + (int64_t)p * 64;
  const IdxAngles an = idx_angles(cs, lane);
  uint16_t *kvr = kv_cache + r * 576;
  reinterpret_cast<i32x4 *>(kvr)[lane] = latent;
  if (lane < 32) {
    float ya, yb;
    rot_pair(bf16_bits_to_f32(tail & 0xffffu), bf16_bits_to_f32(tail >> 16), cs[lane],
             cs[32 + lane], ya, yb);
    reinterpret_cast<uint32_t *>(kvr + 512)[lane] = pack_bf16x2(ya, yb);
  }
  indexer_vec<FP8>(w, an, k_cache + r * 128 * (FP8 ? 1 : 2), FP8 ? k_scale + r : nullptr, lane);
}

// Query side, one workgroup per (row r, part): part rotates indexer heads 16 part .. + 15 (4
// per wave) and a quarter of the MLA heads (one pair per thread and step, in place).  Every
// load of the share is issued before the position is checked and before the first store
// (the outputs may alias the inputs, so the compiler would not hoist them itself).
template <bool FP8>
__device__ __forceinline__ void prep_query_block(int r, int part,
                                                 const int32_t *__restrict__ pos,
                                                 const float *__restrict__ cos_sin, int max_pos,
                                                 const uint16_t *qi_in, uint8_t *qi_out,
                                                 float *__restrict__ qi_scale, int n_heads,
                                                 uint16_t *q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = pos[r];
  const int64_t v0 = (int64_t)r * 64 + 16 * part + 4 * wave;
  uint32_t w[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
    w[hh] = reinterpret_cast<const uint32_t *>(qi_in + (v0 + hh) * 128)[lane];
  const int per_part = (n_heads + 3) / 4;
  const int h0 = part * per_part, h1 = min(n_heads, h0 + per_part);
  const int n_pairs = max(h1 - h0, 0) * 32;
  constexpr int kPairSteps = 4;   // pairs per thread held at once: 32 heads per part
  const int i = threadIdx.x & 31;   // a thread's pairs all use angle i
  uint32_t *pr[kPairSteps];
  uint32_t pv[kPairSteps];
  auto load_pairs = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kPairSteps; ++u) {
      const int j = j0 + u * kPrepThreads + threadIdx.x;
      pr[u] = j < n_pairs ? reinterpret_cast<uint32_t *>(
                                q + ((int64_t)r * n_heads + h0 + (j >> 5)) * 576 + 512) + i
                          : nullptr;
      pv[u] = pr[u] ? *pr[u] : 0u;
    }
  };
  load_pairs(0);
  if (p < 0 || p >= max_pos) return;   // uniform per workgroup
  const float *cs = cos_sin + (int64_t)p * 64;
  const float c = cs[i], sn = cs[32 + i];
  const IdxAngles an = idx_angles(cs, lane);
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
    indexer_vec<FP8>(w[hh], an, qi_out + (v0 + hh) * 128 * (FP8 ? 1 : 2),
                     FP8 ? qi_scale + v0 + hh : nullptr, lane);
  for (int j0 = 0; j0 < n_pairs; j0 += kPairSteps * kPrepThreads) {
    if (j0 > 0) load_pairs(j0);
#pragma unroll
    for (int u = 0; u < kPairSteps; ++u) {
      if (!pr[u]) continue;
      float ya, yb;
      rot_pair(bf16_bits_to_f32(pv[u] & 0xffffu), bf16_bits_to_f32(pv[u] >> 16), c, sn, ya, yb);
      *pr[u] = pack_bf16x2(ya, yb);
    }
  }
}

// One launch for both sides: workgroups [0, 4 R) take the query rows, the rest take the new
// tokens' keys (kPrepWaves tokens each).
template <bool FP8>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    int R, int T, const int32_t *__restrict__ q_pos, const int32_t *__restrict__ k_pos,
    const float *__restrict__ cos_sin, int max_pos, const uint16_t *qi_in, uint8_t *qi_out,
    float *__restrict__ qi_scale, int n_heads, uint16_t *q, const int64_t *__restrict__ rows,
    int64_t cache_rows, const uint16_t *__restrict__ k_in, uint8_t *__restrict__ k_cache,
    float *__restrict__ k_scale, const uint16_t *__restrict__ kv_in,
    uint16_t *__restrict__ kv_cache) {
  const int b = blockIdx.x;
  if (b < 4 * R) {
    prep_query_block<FP8>(b >> 2, b & 3, q_pos, cos_sin, max_pos, qi_in, qi_out, qi_scale,
                          n_heads, q);
    return;
  }
  const int t = (b - 4 * R) * kPrepWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  prep_key_wave<FP8>(t, k_pos, rows, cache_rows, cos_sin, max_pos, k_in, k_cache, k_scale, kv_in,
                     kv_cache, threadIdx.x & 63);
}

hipError_t launch_prep(const PrepQueries &qa, const PrepKeys &ka, const float *cos_sin,
                       int max_pos, bool fp8, hipStream_t stream) {
  const unsigned grid = 4u * (unsigned)qa.R + (unsigned)((ka.T + kPrepWaves - 1) / kPrepWaves);
  if (grid == 0) return hipSuccess;
  const auto *qi = static_cast<const uint16_t *>(qa.qi_in);
  auto *qo = static_cast<uint8_t *>(qa.qi_out);
  auto *qq = static_cast<uint16_t *>(qa.q);
  const auto *ki = static_cast<const uint16_t *>(ka.k_in);
  auto *kc = static_cast<uint8_t *>(ka.k_cache);
  const auto *kvi = static_cast<const uint16_t *>(ka.kv_in);
  auto *kvc = static_cast<uint16_t *>(ka.kv_cache);
  if (fp8)
    prep_kernel<true><<<grid, kPrepThreads, 0, stream>>>(
        qa.R, ka.T, qa.pos, ka.pos, cos_sin, max_pos, qi, qo, qa.qi_scale, qa.n_heads, qq, ka.rows,
        ka.cache_rows, ki, kc, ka.k_scale, kvi, kvc);
  else
    prep_kernel<false><<<grid, kPrepThreads, 0, stream>>>(
        qa.R, ka.T, qa.pos, ka.pos, cos_sin, max_pos, qi, qo, qa.qi_scale, qa.n_heads, qq, ka.rows,
        ka.cache_rows, ki, kc, ka.k_scale, kvi, kvc);
  return hipGetLastError();
}

}  // namespace dsa
