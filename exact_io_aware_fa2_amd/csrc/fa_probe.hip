// fa_probe.hip -- measurement aids, not part of the attention method:
//   * a kernel that only issues bf16 matrix-core products, so a benchmark can report the
//     attention kernels against the throughput this chip actually sustains next to its
//     published peak;
//   * a kernel that only issues float32 atomic adds in the pattern an atomic accumulation
//     of dQ would have (the alternative to the separate dQ pass of the backward), so the
//     choice between the two can be priced with a measured atomic rate.
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

// An atomic dQ would have each key-block workgroup add, for every 32-row step it visits, a
// 32 x 128 float32 tile (its contribution summed over its keys) into a [rows, stride] float32
// accumulator whose rows are `stride` floats apart (Hq * d for a [B, N, Hq, d] layout).
// Each workgroup of 256 threads does that `iters` times, visiting row blocks in a
// pseudo-random order so that many workgroups work on different rows at a time, as the
// workgroups of different key blocks do.  The adds come straight from the accumulator layout
// of v_mfma_f32_32x32x16_bf16 (wave w owns columns 32w..32w+31; register i of lane l holds row
// 8*(i/4) + 4*(l/32) + i%4, column l%32), so each instruction covers two rows of 32
// consecutive floats: the most coalesced form an atomic dQ taken from the MFMA results has.
__global__ __launch_bounds__(256) void atomic_probe_kernel(float* __restrict__ acc,
                                                           int row_blocks, int stride,
                                                           int iters) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int col = w * 32 + (l & 31), r0 = (l >> 5) * 4;
  const float v = 1.f / 1024.f;
  for (int it = 0; it < iters; ++it) {
    const uint32_t rb = ((uint32_t)blockIdx.x * 2654435761u + (uint32_t)it * 40503u) %
                        (uint32_t)row_blocks;
    float* p = acc + (size_t)rb * 32 * stride + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) atomicAdd(p + (size_t)(8 * (i >> 2) + r0 + (i & 3)) * stride, v);
  }
}

hipError_t launch_atomic_probe(float* acc, int row_blocks, int stride, int blocks, int iters,
                               hipStream_t st) {
  hipLaunchKernelGGL(atomic_probe_kernel, dim3(blocks), dim3(256), 0, st, acc, row_blocks,
                     stride, iters);
  return hipGetLastError();
}

}  // namespace fa
