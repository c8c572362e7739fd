// fa_kernels.hpp -- host-side launch interface between the C ABI (fa_api.hip) and the
// kernel files.  Arguments are validated by the caller before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

constexpr float kHostLog2e = 1.4426950408889634f;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d, causal, window;  // packed sequences: B sequences, N = max length
  float c_log2;         // |scale| * log2(e)
  float c_log2_signed;  // scale * log2(e)
  int neg_q;            // 1 when scale < 0 (Q is negated exactly inside the kernel)
  const int* cu;        // packed sequences: B + 1 row offsets (device); null: fixed length
  int ntot;             // packed sequences: rows of the packed tensors
  float o_scale;        // E4M3 forward: the value factor, applied to O in the epilogue
  const float* slopes;  // ALiBi slope per query head (device), or null for no position bias
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;  // D = rowsum(dO * O), laid out like LSE
  int B, Hq, Hkv, N, d, causal, window;  // packed sequences: B sequences, N = max length
  float scale;
  float c_log2_signed;  // scale * log2(e)
  hipEvent_t ev_start;  // optional events recorded around the key-block kernel (may be null)
  hipEvent_t ev_stop;
  const int* cu;        // packed sequences: B + 1 row offsets (device); null: fixed length
  int ntot;             // packed sequences: rows of the packed tensors
  const float* slopes;  // ALiBi slope per query head (device), or null for no position bias
};

struct DecodeArgs {
  const void* q;        // [B, Nq, Hq, d] bf16
  const void* k;        // [B, Nk, Hkv, d] bf16 cache
  const void* v;
  const int* seqlens;   // [B] cached lengths (device), or null: all Nk
  void* o;              // [B, Nq, Hq, d] bf16
  float* lse;           // [B, Hq, Nq]
  float* opart;         // S > 1: [S, B, Hq, Nq, d] float32 partial outputs
  float* lpart;         // S > 1: [S, B, Hq, Nq] partial logsumexps (log2 units)
  int B, Hq, Hkv, Nq, Nk, d, causal, window;
  float c_log2;         // |scale| * log2(e)
  int neg_q;
  int S;                // key chunks per sequence
  hipEvent_t ev_start;  // optional events recorded around the chunk kernel (may be null)
  hipEvent_t ev_stop;
};

// Rows of float32 D the no-allocation backward's static workspace holds (16 MiB).
constexpr size_t kNoAllocRows = (size_t)1 << 22;
// Device address of that workspace on the current device (resolved once per device).
hipError_t noalloc_scratch(float** ptr);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_fwd_fp32(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st);
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st);
hipError_t launch_issue_probe(float* out, int kind, int param, int waves_per_simd, int blocks,
                              int iters, hipStream_t st);
hipError_t launch_fp8_product_probe(const uint8_t* a, const uint8_t* bt, float* c, int sets,
                                    hipStream_t st);
hipError_t launch_atomic_probe(float* acc, int row_blocks, int stride, int blocks, int iters,
                               hipStream_t st);

}  // namespace fa
