// fa_probe.hip -- measurement aids, not part of the attention method:
//   * a kernel that only issues bf16 matrix-core products, so a benchmark can report the
//     attention kernels against the throughput this chip actually sustains next to its
//     published peak;
//   * a kernel that only issues float32 atomic adds in the pattern an atomic accumulation
//     of dQ would have (the alternative to the separate dQ pass of the backward), so the
//     choice between the two can be priced with a measured atomic rate;
//   * issue probes: matrix products next to the other work the attention kernels put
//     beside them (FMAs, exp2, LDS operand reads, operands loaded from global memory) and
//     dependent product chains, to measure how much of that work the matrix core's issue
//     pattern leaves room for.
//   * LDS bank probes: every lane of a wave stores to (or loads from) LDS at lane * stride
//     bytes, so the bank-conflict counters of the launch give the bank count and the lanes
//     served per cycle for each access width (the layouts of the staged tiles rest on them);
//   * a kernel that runs single 32 x 32 x 64 products of 8-bit E4M3 operands given by the
//     caller, so the accuracy of the 8-bit matrix core's 64-term sums can be checked
//     against exact sums (the error bound the 8-bit forward's tolerances rest on).
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

// ---------------------------------------------------------------------------------
// Issue probes.  Every wave runs `iters` rounds of four v_mfma_f32_32x32x16_bf16 products
// (kChains accumulation chains unless stated) and writes one float per lane so that no work
// is optimised away.  The caller sizes the grid (one workgroup of 64 * waves-per-SIMD * 4
// threads per CU for the published figures) and times the launch.

// kind 0 / 1: each product is followed by NV independent FMAs (EXP = false) or v_exp_f32
// (EXP = true) on eight rotating registers; scheduling-group barriers keep the
// interleave (one product, then its NV VALU instructions).
template <int NV, bool EXP>
__global__ __launch_bounds__(512) void issue_valu_kernel(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (int)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * i);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = zero16();
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.01f * (float)((threadIdx.x + i) & 31);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) {
      acc[j] = mfma32(a, b, acc[j]);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int i = (j * NV + v) & 7;
        // exp2 of a value in (0, 1] stays in [0.5, 1]: bounded, never denormal
        x[i] = EXP ? __builtin_amdgcn_exp2f(-x[i]) : __builtin_fmaf(x[i], 0.999f, 0.001f);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // then NV VALU
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 2: eight products per round spread over NCH accumulation chains (NCH = 1: each
// product depends on the one before it).
template <int NCH>
__global__ __launch_bounds__(512) void issue_chain_kernel(float* __restrict__ out, int iters) {
  bf16x8 a[8], b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    b[i] = (__bf16)(0.002f * i);
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j][i] = (__bf16)(0.001f * (int)(threadIdx.x + i + j));
  }
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k % NCH] = mfma32(a[k], b, acc[k % NCH]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 3: NR of each product's operands (A, then B) come from LDS as 16-byte reads
// (consecutive lanes, consecutive 16-byte chunks of a 1 KiB run per wave), issued one
// round ahead into a second register set, as the attention kernels stage their operands.
// The workgroup uses 64 KiB of LDS; every address stays inside it.
constexpr int kIssueLdsBytes = 65536;

// AGPR = true: the accumulators live in AGPRs (assembly products, as the head-dim-256
// kernels hold theirs), so the products' accumulator reads and writes stay out of the VGPRs
// that the LDS reads fill.  RND = true: every operand value (LDS and registers) is drawn
// uniformly from [-2, 2) by a hash of its position, as attention data varies from element
// to element, where the other variants use slowly varying small values.
__device__ __forceinline__ float probe_rnd(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x >> 8) * (4.f / 16777216.f) - 2.f;
}

template <int NR, bool AGPR = false, bool RND = false>
__global__ __launch_bounds__(512) void issue_lds_kernel(float* __restrict__ out, int iters) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // bf16 pairs of small values, so the products stay finite and runs can be compared
  for (int i = t; i < kIssueLdsBytes / 4; i += blockDim.x) {
    const bf16x2 v = RND ? to_bf16x2(probe_rnd(2u * i), probe_rnd(2u * i + 1u))
                         : to_bf16x2(0.001f * (float)(i & 255), 0.002f * (float)(i & 127));
    reinterpret_cast<uint32_t*>(smem)[i] = __builtin_bit_cast(uint32_t, v);
  }
  __syncthreads();
  // byte offset of operand r of chain c in round it: a 1 KiB-aligned run per wave
  auto off = [&](int it, int c, int r) {
    return ((w * 1024 + c * 8192 + r * 4096 + (it & 3) * 2048) & (kIssueLdsBytes - 1024)) +
           lane * 16;
  };
  auto rd = [&](int it, int c, int r) { return lds_read_b128(smem + off(it, c, r)); };
  bf16x8 k0, k1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t id = (uint32_t)(blockIdx.x * blockDim.x + t) * 16u + (uint32_t)i;
    k0[i] = (__bf16)(RND ? probe_rnd(0x40000000u + id) : 0.001f * (int)(t + i));
    k1[i] = (__bf16)(RND ? probe_rnd(0x80000000u + id) : 0.002f * i);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = zero16();
  if constexpr (AGPR) {
    // Wait states between the vector writes of the register operands and of the zeroed
    // accumulators and the first assembly product (the compiler inserts none for inline
    // assembly; without them the first product read stale operands).
    asm volatile("s_nop 4" : "+v"(k0), "+v"(k1));
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) asm volatile("s_nop 4" : "+a"(acc[j]));
  }
  bf16x8 sa[2][kProbeChains], sb[2][kProbeChains];
  auto load = [&](int set, int it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) {
      if (NR >= 1) sa[set][j] = rd(it, j, 0);
      if (NR >= 2) sb[set][j] = rd(it, j, 1);
    }
  };
  auto products = [&](int set) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) {
      const bf16x8& a = NR >= 1 ? sa[set][j] : k0;
      const bf16x8& b = NR >= 2 ? sb[set][j] : k1;
      if constexpr (AGPR) mfma_acc(acc[j], a, b);
      else acc[j] = mfma32(a, b, acc[j]);
    }
  };
  load(0, 0);
  for (int it = 0; it < iters; it += 2) {
    load(1, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    products(0);
    __builtin_amdgcn_sched_barrier(0);
    load(0, it + 2);
    __builtin_amdgcn_sched_barrier(0);
    products(1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (AGPR) {  // the last product's latency before vector reads of the results
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[j]));
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * blockDim.x + t] = s;
}

// kind 6: the A operand of each product read from global memory with 16-byte buffer loads
// (the B operand stays in registers), issued kGlbSets - 1 rounds ahead through a ring of
// register sets, so the load latency is covered as it would be a whole key tile ahead.
// Each workgroup reads a 32 KiB window of `out` (L1 / L2 resident after the first round):
//   MODE 1: each wave reads a 1 KiB run (consecutive lanes, consecutive 16 bytes);
//   MODE 2: the K-operand pattern of the forward kernel: lane (l, h) reads 16 bytes at
//           row l (256-byte rows of a 32-row, 8 KiB tile), byte 16 h + 32 j in round j;
//   MODE 3: chains 0-1 as MODE 2, chains 2-3 read their A operand from LDS one round ahead
//           (half the products with a global operand, half with an LDS one, as a forward
//           with K from global memory and V^T from LDS would have).
// The loads go through a buffer resource that ends at the window, so no address leaves it.
constexpr int kGlbSets = 4;
constexpr uint32_t kGlbWindow = 32768;

template <int MODE>
__global__ __launch_bounds__(512) void issue_glb_kernel(float* __restrict__ out, int iters) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l32 = lane & 31, hh = lane >> 5;
  if constexpr (MODE == 3) {
    for (int i = t; i < kIssueLdsBytes / 4; i += blockDim.x) {
      const bf16x2 v = to_bf16x2(0.001f * (float)(i & 255), 0.002f * (float)(i & 127));
      reinterpret_cast<uint32_t*>(smem)[i] = __builtin_bit_cast(uint32_t, v);
    }
    __syncthreads();
  }
  const uint32_t nwin = (uint32_t)gridDim.x * blockDim.x * 4u / kGlbWindow;  // >= 1 (host)
  const rsrc_t res =
      make_rsrc(reinterpret_cast<const char*>(out) + (size_t)(blockIdx.x % nwin) * kGlbWindow,
                kGlbWindow);
  auto goff = [&](int it, int c) -> uint32_t {
    if constexpr (MODE == 1)
      return (uint32_t)(((w * 1024 + c * 8192 + (it & 3) * 2048) & (int)(kGlbWindow - 1024)) +
                        lane * 16);
    return (uint32_t)(((c + 4 * (it & 1) + w) & 3) * 8192 + l32 * 256 + hh * 16 +
                      ((it >> 1) & 7) * 32);
  };
  auto loff = [&](int it, int c) {
    return ((w * 1024 + c * 8192 + (it & 3) * 2048) & (kIssueLdsBytes - 1024)) + lane * 16;
  };
  constexpr int NG = MODE == 3 ? 2 : kProbeChains;  // chains with a global operand
  bf16x8 k1;
#pragma unroll
  for (int i = 0; i < 8; ++i) k1[i] = (__bf16)(0.002f * i);
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = zero16();
  bf16x8 ga[kGlbSets][NG], la[2][kProbeChains];
  auto gload = [&](int set, int it) {
#pragma unroll
    for (int j = 0; j < NG; ++j) ga[set][j] = __builtin_bit_cast(bf16x8, bload16(res, goff(it, j)));
  };
  auto lload = [&](int set, int it) {
#pragma unroll
    for (int j = NG; j < kProbeChains; ++j) la[set][j] = lds_read_b128(smem + loff(it, j));
  };
  auto products = [&](int gset, int lset) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
      acc[j] = mfma32(j < NG ? ga[gset][j] : la[lset][j], k1, acc[j]);
  };
#pragma unroll
  for (int s2 = 0; s2 < kGlbSets - 1; ++s2) gload(s2, s2);
  if constexpr (MODE == 3) lload(0, 0);
  for (int it = 0; it < iters; it += kGlbSets) {
#pragma unroll
    for (int r = 0; r < kGlbSets; ++r) {
      gload((r + kGlbSets - 1) % kGlbSets, it + r + kGlbSets - 1);
      if constexpr (MODE == 3) lload((r + 1) & 1, it + r + 1);
      __builtin_amdgcn_sched_barrier(0);
      products(r, r & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * blockDim.x + t] = s;
}

// LDS bank probe: every wave of the workgroup accesses 64 KiB of LDS at lane * stride
// bytes (masked to the array and aligned to the access width) `iters` times, with a
// compiler barrier between rounds so every access is issued; W bytes per access.
template <int W, bool STORE>
__global__ __launch_bounds__(512) void lds_bank_kernel(float* __restrict__ out, int stride,
                                                       int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[16384];
  const int t = threadIdx.x, lane = t & 63;
  for (int i = t; i < 16384; i += blockDim.x) buf[i] = i;
  __syncthreads();
  char* base = reinterpret_cast<char*>(buf);
  const uint32_t a = ((uint32_t)lane * (uint32_t)stride) & (65536u - W);
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    if constexpr (STORE) {
      if constexpr (W == 4) *reinterpret_cast<uint32_t*>(base + a) = it;
      if constexpr (W == 8) *reinterpret_cast<uint2*>(base + a) = make_uint2(it, t);
      if constexpr (W == 16) *reinterpret_cast<uint4*>(base + a) = make_uint4(it, t, it, t);
    } else {
      if constexpr (W == 4) acc ^= *reinterpret_cast<const uint32_t*>(base + a);
      if constexpr (W == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(base + a);
        acc ^= v.x ^ v.y;
      }
      if constexpr (W == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + a);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      }
    }
    asm volatile("" ::: "memory");
  }
  __syncthreads();
  out[blockIdx.x * blockDim.x + t] = __uint_as_float(acc ^ buf[(t * 17) & 16383]);
}

template <int W, bool STORE>
static hipError_t launch_lds_bank(int blocks, int threads, float* out, int stride, int iters,
                                  hipStream_t st) {
  hipLaunchKernelGGL((lds_bank_kernel<W, STORE>), dim3(blocks), dim3(threads), 0, st, out,
                     stride, iters);
  return hipGetLastError();
}

template <typename Kernel>
static hipError_t launch_issue(Kernel k, int blocks, int threads, size_t lds, float* out,
                               int iters, hipStream_t st) {
  if (lds > 0) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), lds, st, out, iters);
  return hipGetLastError();
}

hipError_t launch_issue_probe(float* out, int kind, int param, int waves_per_simd, int blocks,
                              int iters, hipStream_t st) {
  const int threads = 256 * waves_per_simd;
  if (kind == 4 || kind == 5) {  // LDS bank probe: param = width * 10000 + stride
    const int width = param / 10000, stride = param % 10000;
    const bool store = kind == 4;
    switch (width * 2 + (store ? 1 : 0)) {
      case 9: return launch_lds_bank<4, true>(blocks, threads, out, stride, iters, st);
      case 8: return launch_lds_bank<4, false>(blocks, threads, out, stride, iters, st);
      case 17: return launch_lds_bank<8, true>(blocks, threads, out, stride, iters, st);
      case 16: return launch_lds_bank<8, false>(blocks, threads, out, stride, iters, st);
      case 33: return launch_lds_bank<16, true>(blocks, threads, out, stride, iters, st);
      case 32: return launch_lds_bank<16, false>(blocks, threads, out, stride, iters, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (kind * 100 + param) {
    case 0: return launch_issue(issue_valu_kernel<0, false>, blocks, threads, 0, out, iters, st);
    case 2: return launch_issue(issue_valu_kernel<2, false>, blocks, threads, 0, out, iters, st);
    case 4: return launch_issue(issue_valu_kernel<4, false>, blocks, threads, 0, out, iters, st);
    case 6: return launch_issue(issue_valu_kernel<6, false>, blocks, threads, 0, out, iters, st);
    case 8: return launch_issue(issue_valu_kernel<8, false>, blocks, threads, 0, out, iters, st);
    case 12: return launch_issue(issue_valu_kernel<12, false>, blocks, threads, 0, out, iters, st);
    case 101: return launch_issue(issue_valu_kernel<1, true>, blocks, threads, 0, out, iters, st);
    case 102: return launch_issue(issue_valu_kernel<2, true>, blocks, threads, 0, out, iters, st);
    case 103: return launch_issue(issue_valu_kernel<3, true>, blocks, threads, 0, out, iters, st);
    case 104: return launch_issue(issue_valu_kernel<4, true>, blocks, threads, 0, out, iters, st);
    case 106: return launch_issue(issue_valu_kernel<6, true>, blocks, threads, 0, out, iters, st);
    case 108: return launch_issue(issue_valu_kernel<8, true>, blocks, threads, 0, out, iters, st);
    case 201: return launch_issue(issue_chain_kernel<1>, blocks, threads, 0, out, iters, st);
    case 202: return launch_issue(issue_chain_kernel<2>, blocks, threads, 0, out, iters, st);
    case 204: return launch_issue(issue_chain_kernel<4>, blocks, threads, 0, out, iters, st);
    case 208: return launch_issue(issue_chain_kernel<8>, blocks, threads, 0, out, iters, st);
    case 300: return launch_issue(issue_lds_kernel<0>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 301: return launch_issue(issue_lds_kernel<1>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 302: return launch_issue(issue_lds_kernel<2>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 310: return launch_issue(issue_lds_kernel<0, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 311: return launch_issue(issue_lds_kernel<1, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 312: return launch_issue(issue_lds_kernel<2, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 320: return launch_issue(issue_lds_kernel<0, false, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 321: return launch_issue(issue_lds_kernel<1, false, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 322: return launch_issue(issue_lds_kernel<2, false, true>, blocks, threads, kIssueLdsBytes, out, iters, st);
    case 601: return launch_issue(issue_glb_kernel<1>, blocks, threads, 0, out, iters, st);
    case 602: return launch_issue(issue_glb_kernel<2>, blocks, threads, 0, out, iters, st);
    case 603: return launch_issue(issue_glb_kernel<3>, blocks, threads, kIssueLdsBytes, out, iters, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------------
// 8-bit product probe: wave w of workgroup g computes set 4 g + w, C = A B with
// A[m][k] = a[set][m][k] and B[k][n] = bt[set][n][k] (32 x 64 codes each, row-major per set),
// as one v_mfma_f32_32x32x64_f8f6f4 from a zero accumulator, and writes C[m][n] as float32
// to c[set][m][n].  Lane l holds row / column l % 32 of each operand and its 32 bytes
// k = 32 (l / 32) + byte; the result is in the accumulator layout of the bf16 product.
typedef int i32x8p __attribute__((ext_vector_type(8)));
typedef float f32v16p __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void fp8_product_kernel(const uint8_t* __restrict__ a,
                                                          const uint8_t* __restrict__ bt,
                                                          float* __restrict__ c, int sets) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int set = blockIdx.x * 4 + w;
  if (set >= sets) return;  // whole wave
  const size_t base = (size_t)set * 2048 + (size_t)(l & 31) * 64 + 32 * (l >> 5);
  const uint4 a0 = *reinterpret_cast<const uint4*>(a + base);
  const uint4 a1 = *reinterpret_cast<const uint4*>(a + base + 16);
  const uint4 b0 = *reinterpret_cast<const uint4*>(bt + base);
  const uint4 b1 = *reinterpret_cast<const uint4*>(bt + base + 16);
  const i32x8p ao = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                     (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8p bo = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  f32v16p z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  const f32v16p r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ao, bo, z, 0, 0, 0, 0, 0, 0);
  float* cs = c + (size_t)set * 1024;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = 8 * (i >> 2) + 4 * (l >> 5) + (i & 3), n = l & 31;
    cs[m * 32 + n] = r[i];
  }
}

hipError_t launch_fp8_product_probe(const uint8_t* a, const uint8_t* bt, float* c, int sets,
                                    hipStream_t st) {
  hipLaunchKernelGGL(fp8_product_kernel, dim3((sets + 3) / 4), dim3(256), 0, st, a, bt, c, sets);
  return hipGetLastError();
}

}  // namespace fa
