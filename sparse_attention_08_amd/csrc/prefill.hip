// prefill.hip -- the prefill attention of DSA with its dispatch between the two ways the pages
// run it ("DeepSeek-V3.2 技术报告摘要", section 1: MLA in MQA mode over the top-k entries,
// and "短序列优化": short prefill as masked MHA; the switch length is the serving knob of
// "DeepSeek-V3.2" model docs, section 5.3, SGLANG_NSA_PREFILL_DENSE_ATTN_KV_LEN_THRESHOLD).
//
// Both ways take the per-head query [q_nope (128) | q_rope (64)] and the latent cache, and
// return per-head 128-dim values.  The MQA way works in the latent space: it absorbs W_UK
// into the query, q_abs[r, h] = [W_UK[h]^T q_nope[r, h] (512) | q_rope[r, h] (64)], attends
// with the sparse MLA over the top-k entries (values: the 512 latent dims), and maps the
// result back through W_UV, out[r, h] = W_UV[h] o[r, h].  Both products are gemm_nt.h
// problems; W_UK is transposed once per call so its contraction dim (d) is contiguous.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "gemm_nt.h"

namespace dsa {

// W_UK [H][128][512] -> W_UK^T [H][512][128] through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void transpose_wuk_kernel(const uint16_t *__restrict__ w,
                                                            uint16_t *__restrict__ wt) {
  __shared__ uint16_t tile[32][33];
  const int h = blockIdx.z, d0 = blockIdx.y * 32, k0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  const uint16_t *src = w + (int64_t)h * 128 * 512;
  uint16_t *dst = wt + (int64_t)h * 512 * 128;
  for (int j = ty; j < 32; j += 8) tile[j][tx] = src[(int64_t)(d0 + j) * 512 + k0 + tx];
  __syncthreads();
  for (int j = ty; j < 32; j += 8) dst[(int64_t)(k0 + j) * 128 + d0 + tx] = tile[tx][j];
}

// q_rope of every (row, head) into the last 64 dims of q_abs: 8 lanes x 16 bytes per pair.
__global__ __launch_bounds__(256) void copy_rope_kernel(const uint16_t *__restrict__ q,
                                                        uint16_t *__restrict__ q_abs, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (pair, 16-byte piece)
  if (i >= n * 8) return;
  const int64_t pr = i >> 3;
  const int piece = (int)(i & 7);
  *reinterpret_cast<i32x4 *>(q_abs + pr * 576 + 512 + 8 * piece) =
      *reinterpret_cast<const i32x4 *>(q + pr * 192 + 128 + 8 * piece);
}

// q_abs[r, h, 0:512] = W_UK[h]^T q_nope[r, h]: batch z = head, A row m = q_nope of (m, z),
// B row n = row n of W_UK^T[z], C row m = q_abs of (m, z).
struct AbsorbProb {
  int M, N, K, H;
  const uint16_t *q, *wt;
  uint16_t *q_abs;
  __device__ GemmRow a(int m, int z) const { return {q + ((int64_t)m * H + z) * 192, true}; }
  __device__ const uint16_t *b(int n, int z) const { return wt + ((int64_t)z * 512 + n) * 128; }
  __device__ uint16_t *c(int m, int z) const { return q_abs + ((int64_t)m * H + z) * 576; }
};

// out[r, h] = W_UV[h] o[r, h]: A row m = o of (m, z) (512), B row n = W_UV[z] row n.
struct ExpandProb {
  int M, N, K, H;
  const uint16_t *o, *w;
  uint16_t *out;
  __device__ GemmRow a(int m, int z) const { return {o + ((int64_t)m * H + z) * 512, true}; }
  __device__ const uint16_t *b(int n, int z) const { return w + ((int64_t)z * 128 + n) * 512; }
  __device__ uint16_t *c(int m, int z) const { return out + ((int64_t)m * H + z) * 128; }
};

namespace {
size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t absorb_workspace_bytes(int R, int H) {
  return a256((size_t)H * 512 * 128 * 2) + a256((size_t)R * H * 576 * 2) +
         a256((size_t)R * H * 512 * 2);
}

AbsorbBuffers carve_absorb(void *ws, int R, int H) {
  uint8_t *p = static_cast<uint8_t *>(ws);
  AbsorbBuffers b;
  b.wuk_t = reinterpret_cast<uint16_t *>(p);
  p += a256((size_t)H * 512 * 128 * 2);
  b.q_abs = reinterpret_cast<uint16_t *>(p);
  p += a256((size_t)R * H * 576 * 2);
  b.o_lat = reinterpret_cast<uint16_t *>(p);
  return b;
}

hipError_t launch_absorb_query(int R, int H, const void *q, const void *w_uk,
                               const AbsorbBuffers &b, hipStream_t stream) {
  const auto *q16 = static_cast<const uint16_t *>(q);
  transpose_wuk_kernel<<<dim3(512 / 32, 128 / 32, H), 256, 0, stream>>>(
      static_cast<const uint16_t *>(w_uk), b.wuk_t);
  const int64_t pairs = (int64_t)R * H;
  copy_rope_kernel<<<(unsigned)((pairs * 8 + 255) / 256), 256, 0, stream>>>(q16, b.q_abs, pairs);
  const AbsorbProb pr{R, 512, 128, H, q16, b.wuk_t, b.q_abs};
  gemm_nt_kernel<<<dim3(512 / kGemmTile, (R + kGemmTileM - 1) / kGemmTileM, H), kGemmThreads, 0,
                   stream>>>(pr);
  return hipGetLastError();
}

hipError_t launch_expand_output(int R, int H, const uint16_t *o_lat, const void *w_uv, void *out,
                                hipStream_t stream) {
  const ExpandProb pr{R, 128, 512, H, o_lat, static_cast<const uint16_t *>(w_uv),
                      static_cast<uint16_t *>(out)};
  gemm_nt_kernel<<<dim3(1, (R + kGemmTileM - 1) / kGemmTileM, H), kGemmThreads, 0, stream>>>(pr);
  return hipGetLastError();
}

}  // namespace dsa
