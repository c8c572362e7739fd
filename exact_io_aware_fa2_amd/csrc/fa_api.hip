// fa_api.hip -- the extern "C" boundary of libfa.so (declared in include/fa.h).
//
// Every entry point validates its arguments on the host before enqueuing anything, never
// allocates or synchronises, and reports failures through a status code plus a
// thread-local message.
#include <math.h>

#include <algorithm>
#include <initializer_list>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_kernels.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_time_start = nullptr;  // pending fa_bwd_time_main_kernel request
thread_local hipEvent_t g_time_stop = nullptr;

fa_status fail(fa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

fa_status ok() {
  g_err[0] = '\0';
  return FA_OK;
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // kernels index rows with 32-bit ints
constexpr int kMaxSplits = 256;                  // key chunks per sequence in fa_decode

// Product of non-negative factors, saturated at kMaxElems: never overflows, whatever int
// sizes a caller passes (every partial product stays below 2^31 before the next factor).
int64_t sat_mul(std::initializer_list<int64_t> xs) {
  int64_t p = 1;
  for (int64_t x : xs) {
    if (x <= 0) return 0;
    if (x >= kMaxElems || p >= kMaxElems / x + 1) return kMaxElems;
    p *= x;
    if (p >= kMaxElems) return kMaxElems;
  }
  return p;
}

fa_status check_common(const char* fn, int B, int Hq, int Hkv, int N, int d, int causal,
                       int window, float scale) {
  (void)causal;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
    return fail(FA_ERR_INVALID_ARG, "%s: sizes must be positive (B=%d Hq=%d Hkv=%d N=%d d=%d)",
                fn, B, Hq, Hkv, N, d);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (window < 0) return fail(FA_ERR_INVALID_ARG, "%s: window=%d must be >= 0", fn, window);
  if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (d != 64 && d != 128 && d != 256)
    return fail(FA_ERR_UNSUPPORTED, "%s: head dim %d not supported (64, 128 or 256)", fn, d);
  if (sat_mul({B, N, Hq, d}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "%s: B*N*Hq*d = %.4g elements reaches 2^31", fn,
                (double)B * N * Hq * d);
  return FA_OK;
}

fa_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return ok();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tensors move through 16-byte vector loads and stores; the float32 row statistics and the
// int32 / float32 side arrays through 4-byte ones.  (Null optional pointers pass.)
bool misaligned(std::initializer_list<const void*> ptrs, uintptr_t bytes) {
  for (const void* p : ptrs)
    if (((uintptr_t)p & (bytes - 1)) != 0) return true;
  return false;
}
fa_status check_align(const char* fn, std::initializer_list<const void*> t16,
                      std::initializer_list<const void*> t4) {
  if (misaligned(t16, 16) || misaligned(t4, 4))
    return fail(FA_ERR_INVALID_ARG,
                "%s: tensor pointers must be 16-byte aligned (row statistics and side arrays "
                "4-byte aligned)", fn);
  return FA_OK;
}

// Packed sequences: the shared checks on (Hq, Hkv, d, window, scale) run as for one batch
// entry of `total` rows; on top, the offsets pointer, counts and grid size are checked.
// The offsets themselves live on the device and are not read here (the kernels clamp
// them into the tensors).
fa_status check_varlen(const char* fn, const int* cu, int num_seqs, int total, int max_seqlen,
                       int Hq, int Hkv, int d, int causal, int window, float scale) {
  if (!cu) return fail(FA_ERR_INVALID_ARG, "%s: null cu_seqlens", fn);
  if (num_seqs <= 0 || total <= 0 || max_seqlen <= 0)
    return fail(FA_ERR_INVALID_ARG, "%s: num_seqs=%d, total=%d, max_seqlen=%d must be positive",
                fn, num_seqs, total, max_seqlen);
  if (max_seqlen > total)
    return fail(FA_ERR_INVALID_ARG, "%s: max_seqlen=%d exceeds total=%d", fn, max_seqlen, total);
  fa_status st = check_common(fn, 1, Hq, Hkv, total, d, causal, window, scale);
  if (st != FA_OK) return st;
  if (sat_mul({num_seqs, Hq, (max_seqlen + 31) / 32}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "%s: num_seqs * Hq * max_seqlen too large for one grid", fn);
  return FA_OK;
}

// The bf16 forward behind fa_fwd and fa_fwd_alibi (slopes == nullptr: no position bias).
fa_status fwd_bf16(const char* fn, const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int N, int d, int causal, int window,
                   float scale, const float* slopes, void* stream) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "%s: null pointer", fn);
  fa_status st = check_common(fn, B, Hq, Hkv, N, d, causal, window, scale);
  if (st == FA_OK) st = check_align(fn, {q, k, v, o}, {lse, slopes});
  if (st != FA_OK) return st;
  // The bf16 kernel works with the non-negative log2 scale |scale| log2(e) (a negative scale
  // negates Q exactly) and marks masked scores with -inf; for scale == 0 it gets a tiny
  // positive value instead of 0 so that -inf * scale stays -inf (every unmasked weight still
  // rounds to exactly 1).
  const float c2 = scale == 0.f ? 1e-30f : fabsf(scale) * fa::kHostLog2e;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal ? 1 : 0, window, c2,
                scale * fa::kHostLog2e, scale < 0.f ? 1 : 0};
  a.slopes = slopes;
  return launched(fn, fa::launch_fwd_bf16(a, (hipStream_t)stream));
}

fa_status bwd_bf16(const char* fn, const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                   int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                   void* workspace, size_t workspace_bytes, const float* slopes,
                   void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "%s: null pointer", fn);
  fa_status st = check_common(fn, B, Hq, Hkv, N, d, causal, window, scale);
  if (st == FA_OK) st = check_align(fn, {q, k, v, o, dO, dq, dk, dv}, {lse, slopes});
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_size(B, Hq, Hkv, N, d, causal, window);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(FA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  fa::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv,
                N, d, causal ? 1 : 0, window, scale, scale * fa::kHostLog2e, g_time_start,
                g_time_stop};
  g_time_start = g_time_stop = nullptr;
  a.slopes = slopes;
  return launched(fn, fa::launch_bwd_bf16(a, (hipStream_t)stream));
}

fa_status fwd_varlen(const char* fn, const void* q, const void* k, const void* v, void* o,
                     float* lse, const int* cu_seqlens, int num_seqs, int total,
                     int max_seqlen, int Hq, int Hkv, int d, int causal, int window,
                     float scale, const float* slopes, void* stream) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "%s: null pointer", fn);
  fa_status st = check_varlen(fn, cu_seqlens, num_seqs, total, max_seqlen, Hq, Hkv, d, causal,
                              window, scale);
  if (st == FA_OK) st = check_align(fn, {q, k, v, o}, {lse, cu_seqlens, slopes});
  if (st != FA_OK) return st;
  const float c2 = scale == 0.f ? 1e-30f : fabsf(scale) * fa::kHostLog2e;  // as in fwd_bf16
  fa::FwdArgs a{q, k, v, o, lse, num_seqs, Hq, Hkv, max_seqlen, d, causal ? 1 : 0, window,
                c2, scale * fa::kHostLog2e, scale < 0.f ? 1 : 0, cu_seqlens, total};
  a.slopes = slopes;
  return launched(fn, fa::launch_fwd_bf16(a, (hipStream_t)stream));
}

fa_status bwd_varlen(const char* fn, const void* q, const void* k, const void* v,
                     const void* o, const void* dO, const float* lse, void* dq, void* dk,
                     void* dv, const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                     int Hq, int Hkv, int d, int causal, int window, float scale,
                     void* workspace, size_t workspace_bytes, const float* slopes,
                     void* stream) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "%s: null pointer", fn);
  fa_status st = check_varlen(fn, cu_seqlens, num_seqs, total, max_seqlen, Hq, Hkv, d, causal,
                              window, scale);
  if (st == FA_OK)
    st = check_align(fn, {q, k, v, o, dO, dq, dk, dv}, {lse, cu_seqlens, slopes});
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_varlen_workspace_size(total, Hq, Hkv, d);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(FA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  fa::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, static_cast<float*>(workspace), num_seqs, Hq,
                Hkv, max_seqlen, d, causal ? 1 : 0, window, scale, scale * fa::kHostLog2e,
                g_time_start, g_time_stop, cu_seqlens, total};
  g_time_start = g_time_stop = nullptr;
  a.slopes = slopes;
  return launched(fn, fa::launch_bwd_bf16(a, (hipStream_t)stream));
}

// The *_alibi entry points require their slope array.
fa_status need_slopes(const char* fn, const float* slopes) {
  if (!slopes)
    return fail(FA_ERR_INVALID_ARG, "%s: null alibi_slopes (use the plain entry point for no "
                "position bias)", fn);
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                 void* stream) {
  return fwd_bf16("fa_fwd", q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, nullptr,
                  stream);
}

fa_status fa_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                       const float* alibi_slopes, void* stream) {
  const fa_status st = need_slopes("fa_fwd_alibi", alibi_slopes);
  if (st != FA_OK) return st;
  return fwd_bf16("fa_fwd_alibi", q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale,
                  alibi_slopes, stream);
}

fa_status fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                      int B, int Hq, int Hkv, int N, int d, int causal, int window,
                      float scale, void* stream) {
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp32: null pointer");
  fa_status st = check_common("fa_fwd_fp32", B, Hq, Hkv, N, d, causal, window, scale);
  if (st == FA_OK) st = check_align("fa_fwd_fp32", {q, k, v, o}, {lse});
  if (st != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal ? 1 : 0, window,
                fabsf(scale) * fa::kHostLog2e, scale * fa::kHostLog2e, 0};
  return launched("fa_fwd_fp32", fa::launch_fwd_fp32(a, (hipStream_t)stream));
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     float descale_q, float descale_k, float descale_v, int B, int Hq, int Hkv,
                     int N, int d, int causal, int window, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: null pointer");
  fa_status st = check_common("fa_fwd_fp8", B, Hq, Hkv, N, d, causal, window, scale);
  if (st == FA_OK) st = check_align("fa_fwd_fp8", {q, k, v, o}, {lse});
  if (st != FA_OK) return st;
  if (!(isfinite(descale_q) && descale_q > 0.f && isfinite(descale_k) && descale_k > 0.f &&
        isfinite(descale_v) && descale_v > 0.f))
    return fail(FA_ERR_INVALID_ARG,
                "fa_fwd_fp8: dequantisation factors must be finite and positive (%g, %g, %g)",
                (double)descale_q, (double)descale_k, (double)descale_v);
  // The kernel multiplies the raw code products by |scale| dq dk log2(e) (a negative scale
  // negates Q exactly); a product that underflows is replaced by a tiny positive value so
  // that masked scores stay -inf, as in fa_fwd.
  const double cd = fabs((double)scale) * descale_q * descale_k * 1.4426950408889634;
  if (!(cd < 3.0e38))
    return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: |scale| * descale_q * descale_k too large");
  const float c2 = cd < 1e-30 ? 1e-30f : (float)cd;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal ? 1 : 0, window, c2, 0.f,
                scale < 0.f ? 1 : 0, nullptr, 0, descale_v};
  return launched("fa_fwd_fp8", fa::launch_fwd_fp8(a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal, int window) {
  if (check_common("fa_bwd_workspace_size", B, Hq, Hkv, N, d, causal, window, 1.f) != FA_OK)
    return 0;
  return align256((size_t)B * Hq * N * sizeof(float));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                 int N, int d, int causal, int window, float scale, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return bwd_bf16("fa_bwd", q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window,
                  scale, workspace, workspace_bytes, nullptr, stream);
}

fa_status fa_bwd_alibi(const void* q, const void* k, const void* v, const void* o,
                       const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                       int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                       void* workspace, size_t workspace_bytes, const float* alibi_slopes,
                       void* stream) {
  const fa_status st = need_slopes("fa_bwd_alibi", alibi_slopes);
  if (st != FA_OK) return st;
  return bwd_bf16("fa_bwd_alibi", q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal,
                  window, scale, workspace, workspace_bytes, alibi_slopes, stream);
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int N, int d, int causal, int window, float scale,
                         void* stream) {
  static const char* fn = "fa_bwd_noalloc";
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARG, "%s: null pointer", fn);
  fa_status st = check_common(fn, B, Hq, Hkv, N, d, causal, window, scale);
  if (st != FA_OK) return st;
  if (sat_mul({B, Hq, N}) > (int64_t)fa::kNoAllocRows)
    return fail(FA_ERR_WORKSPACE,
                "%s: B*Hq*N = %lld rows exceed the %zu rows of its static workspace (use "
                "fa_bwd with a caller workspace)", fn, (long long)B * Hq * N, fa::kNoAllocRows);
  float* ws = nullptr;
  const hipError_t e = fa::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "%s: static workspace address: HIP error %d (%s)", fn, (int)e,
                hipGetErrorString(e));
  return bwd_bf16(fn, q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
                  ws, fa::kNoAllocRows * sizeof(float), nullptr, stream);
}

fa_status fa_mfma_probe(float* out, int blocks, int iters, void* stream) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "fa_mfma_probe: null pointer");
  if (blocks <= 0 || iters <= 0)
    return fail(FA_ERR_INVALID_ARG, "fa_mfma_probe: blocks and iters must be positive");
  return launched("fa_mfma_probe", fa::launch_mfma_probe(out, blocks, iters, (hipStream_t)stream));
}

fa_status fa_atomic_probe(float* acc, int row_blocks, int stride, int blocks, int iters,
                          void* stream) {
  if (!acc) return fail(FA_ERR_INVALID_ARG, "fa_atomic_probe: null pointer");
  if (row_blocks <= 0 || stride < 128 || blocks <= 0 || iters <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "fa_atomic_probe: row_blocks, blocks and iters must be positive, stride >= 128");
  if (sat_mul({row_blocks, 32, stride}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "fa_atomic_probe: row_blocks * 32 * stride reaches 2^31");
  return launched("fa_atomic_probe", fa::launch_atomic_probe(acc, row_blocks, stride, blocks,
                                                             iters, (hipStream_t)stream));
}

// The (kind, param) pairs fa_issue_probe has kernels for.
static bool issue_probe_supported(int kind, int param) {
  switch (kind) {
    case 0: return param == 0 || param == 2 || param == 4 || param == 6 || param == 8 || param == 12;
    case 1: return param == 1 || param == 2 || param == 3 || param == 4 || param == 6 || param == 8;
    case 2: return param == 1 || param == 2 || param == 4 || param == 8;
    case 3: return (param >= 0 && param <= 2) || (param >= 10 && param <= 12) ||
                   (param >= 20 && param <= 22);
    case 6: return param == 1 || param == 2 || param == 3;
    case 4:
    case 5: {  // LDS bank probe: width * 10000 + stride
      const int width = param / 10000, stride = param % 10000;
      return (width == 4 || width == 8 || width == 16) && stride >= 1 && stride <= 4096;
    }
    default: return false;
  }
}

fa_status fa_issue_probe(float* out, int kind, int param, int waves_per_simd, int blocks,
                         int iters, void* stream) {
  if (!out) return fail(FA_ERR_INVALID_ARG, "fa_issue_probe: null pointer");
  if (!issue_probe_supported(kind, param))
    return fail(FA_ERR_UNSUPPORTED, "fa_issue_probe: unsupported (kind, param)");
  if ((waves_per_simd != 1 && waves_per_simd != 2) || blocks <= 0 || iters <= 0)
    return fail(FA_ERR_INVALID_ARG,
                "fa_issue_probe: waves_per_simd must be 1 or 2, blocks and iters positive");
  if (kind == 6 && blocks * waves_per_simd < 32)  // `out` must hold one 32 KiB read window
    return fail(FA_ERR_INVALID_ARG, "fa_issue_probe: kind 6 needs blocks * waves_per_simd >= 32");
  return launched("fa_issue_probe", fa::launch_issue_probe(out, kind, param, waves_per_simd,
                                                           blocks, iters, (hipStream_t)stream));
}

fa_status fa_fp8_product_probe(const void* a, const void* bt, float* c, int sets,
                               void* stream) {
  if (!a || !bt || !c) return fail(FA_ERR_INVALID_ARG, "fa_fp8_product_probe: null pointer");
  if (sets <= 0) return fail(FA_ERR_INVALID_ARG, "fa_fp8_product_probe: sets must be positive");
  if (sat_mul({sets, 2048}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "fa_fp8_product_probe: sets * 2048 reaches 2^31");
  if (misaligned({a, bt}, 16) || misaligned({c}, 4))
    return fail(FA_ERR_INVALID_ARG, "fa_fp8_product_probe: misaligned pointer");
  return launched("fa_fp8_product_probe",
                  fa::launch_fp8_product_probe(static_cast<const uint8_t*>(a),
                                               static_cast<const uint8_t*>(bt), c, sets,
                                               (hipStream_t)stream));
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int Hq,
                        int Hkv, int d, int causal, int window, float scale, void* stream) {
  return fwd_varlen("fa_fwd_varlen", q, k, v, o, lse, cu_seqlens, num_seqs, total, max_seqlen,
                    Hq, Hkv, d, causal, window, scale, nullptr, stream);
}

fa_status fa_fwd_varlen_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                              int Hq, int Hkv, int d, int causal, int window, float scale,
                              const float* alibi_slopes, void* stream) {
  const fa_status st = need_slopes("fa_fwd_varlen_alibi", alibi_slopes);
  if (st != FA_OK) return st;
  return fwd_varlen("fa_fwd_varlen_alibi", q, k, v, o, lse, cu_seqlens, num_seqs, total,
                    max_seqlen, Hq, Hkv, d, causal, window, scale, alibi_slopes, stream);
}

size_t fa_bwd_varlen_workspace_size(int total, int Hq, int Hkv, int d) {
  if (total <= 0 || check_common("fa_bwd_varlen_workspace_size", 1, Hq, Hkv, total, d, 0, 0,
                                 1.f) != FA_OK)
    return 0;
  return align256((size_t)Hq * total * sizeof(float));
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse, void* dq, void* dk, void* dv,
                        const int* cu_seqlens, int num_seqs, int total, int max_seqlen, int Hq,
                        int Hkv, int d, int causal, int window, float scale, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return bwd_varlen("fa_bwd_varlen", q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens, num_seqs,
                    total, max_seqlen, Hq, Hkv, d, causal, window, scale, workspace,
                    workspace_bytes, nullptr, stream);
}

fa_status fa_bwd_varlen_alibi(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int num_seqs, int total, int max_seqlen,
                              int Hq, int Hkv, int d, int causal, int window, float scale,
                              void* workspace, size_t workspace_bytes,
                              const float* alibi_slopes, void* stream) {
  const fa_status st = need_slopes("fa_bwd_varlen_alibi", alibi_slopes);
  if (st != FA_OK) return st;
  return bwd_varlen("fa_bwd_varlen_alibi", q, k, v, o, dO, lse, dq, dk, dv, cu_seqlens,
                    num_seqs, total, max_seqlen, Hq, Hkv, d, causal, window, scale, workspace,
                    workspace_bytes, alibi_slopes, stream);
}

int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || Hq % Hkv != 0 ||
      (d != 64 && d != 128) || num_splits < 0 || num_splits > kMaxSplits)
    return 0;
  if (num_splits > 0) return num_splits;
  // About one workgroup per compute unit (256 units; measured faster than two per unit,
  // with a shorter merge), chunks of at least 256 keys.
  const int64_t nrg = ((int64_t)(Hq / Hkv) * Nq + 31) / 32;  // < 2^58: no overflow
  const int64_t base = sat_mul({B, Hkv, nrg});
  int64_t s = (256 + base - 1) / base;
  s = std::min<int64_t>(s, std::max(1, Nk / 256));
  s = std::min<int64_t>(s, 64);
  return (int)std::max<int64_t>(s, 1);
}

size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
  const int S = fa_decode_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (S <= 1) return 0;
  // fa_decode accepts only B * Nq * Hq * d < 2^31, so the partial outputs of S <= 256 chunks
  // stay far below size_t's range; larger sizes report 0 (the call itself would be rejected)
  if (sat_mul({B, Nq, Hq, d}) >= kMaxElems) return 0;
  const size_t rows = (size_t)S * B * Hq * Nq;
  return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int* seqlens_k, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                    int Nk, int d, int causal, int window, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !o || !lse)
    return fail(FA_ERR_INVALID_ARG, "fa_decode: null pointer");
  if (Nq <= 0) return fail(FA_ERR_INVALID_ARG, "fa_decode: Nq=%d must be positive", Nq);
  fa_status st = check_common("fa_decode", B, Hq, Hkv, Nk, d, causal, window, scale);
  if (st == FA_OK) st = check_align("fa_decode", {q, k_cache, v_cache, o}, {lse, seqlens_k});
  if (st != FA_OK) return st;
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode: head dim %d not supported (64 or 128)", d);
  if (sat_mul({B, Nq, Hq, d}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "fa_decode: B*Nq*Hq*d reaches 2^31");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(FA_ERR_INVALID_ARG, "fa_decode: num_splits=%d outside [0, %d]", num_splits,
                kMaxSplits);
  const int S = fa_decode_num_splits(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (sat_mul({B, Hkv, ((int64_t)(Hq / Hkv) * Nq + 31) / 32, S}) >= kMaxElems)
    return fail(FA_ERR_INVALID_ARG, "fa_decode: grid too large");
  const size_t need = fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_WORKSPACE, "fa_decode: workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && ((uintptr_t)workspace & 255) != 0)
    return fail(FA_ERR_WORKSPACE, "fa_decode: workspace must be 256-byte aligned");
  const float c2 = scale == 0.f ? 1e-30f : fabsf(scale) * fa::kHostLog2e;  // as in fa_fwd
  fa::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens_k;
  a.o = o;
  a.lse = lse;
  if (S > 1) {
    const size_t rows = (size_t)S * B * Hq * Nq;
    a.opart = static_cast<float*>(workspace);
    a.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align256(rows * d * sizeof(float)));
  }
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal ? 1 : 0;
  a.window = window;
  a.c_log2 = c2;
  a.neg_q = scale < 0.f ? 1 : 0;
  a.S = S;
  a.ev_start = g_time_start;
  a.ev_stop = g_time_stop;
  g_time_start = g_time_stop = nullptr;
  return launched("fa_decode", fa::launch_decode(a, (hipStream_t)stream));
}

fa_status fa_bwd_time_main_kernel(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(FA_ERR_INVALID_ARG, "fa_bwd_time_main_kernel: give both events or neither");
  g_time_start = static_cast<hipEvent_t>(start_event);
  g_time_stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

const char* fa_last_error(void) { return g_err; }

const char* fa_version(void) { return "libfa 0.1.0 (gfx950)"; }

}  // extern "C"
