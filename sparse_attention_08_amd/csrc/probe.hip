// probe.hip -- a measurement aid: the bf16 matrix-core rate the GPU sustains (the kernel
// rooflines are stated against the published peak; this measures what the chip delivers at
// the clock it holds under a pure MFMA load).  Not a step of the method.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "dsa.h"

namespace dsa {

constexpr int kProbeThreads = 256;   // 4 waves: one per SIMD; two workgroups per CU
constexpr int kProbeBlocks = DSA_MFMA_PROBE_WAVES / (kProbeThreads / kWave);   // 512

// The register budget of 4+ waves per SIMD keeps the accumulators in ordinary registers: the
// loop is then the 8 products alone (with the full budget the compiler moves the accumulators
// through the accumulation registers every iteration).
__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void
mfma_rate_kernel(int iters, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  // operands that the compiler cannot fold: built from the lane id
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (lane == 0) out[blockIdx.x * (kProbeThreads / kWave) + (threadIdx.x >> 6)] = s;
}

}  // namespace dsa

extern "C" int dsa_mfma_rate_probe(int iters, float *out, void *stream) {
  if (iters < 1 || iters > 1000000 || !out) return DSA_ERR_INVALID_ARG;
  dsa::mfma_rate_kernel<<<dsa::kProbeBlocks, dsa::kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      iters, out);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}
