// fa_probe.hip -- a measurement aid, not part of the attention method: a kernel that only
// issues bf16 matrix-core products, so a benchmark can report the attention kernels
// against the throughput this chip actually sustains next to its published peak.
#include <hip/hip_runtime.h>

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

// Each wave runs kChains independent accumulation chains of v_mfma_f32_32x32x16_bf16 for
// `iters` rounds and writes one float per lane (so the products are not optimised away).
constexpr int kProbeChains = 4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((threadIdx.x & 7) * 0.125f + i);
    b[i] = (__bf16)(i * 0.5f - 1.f);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace fa
