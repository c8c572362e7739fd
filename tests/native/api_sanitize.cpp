// Driver of the sanitizer build of the C ABI layer (tests/test_abi.py builds it with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side only, linked with the
// recording launchers of stub_launchers.cpp).  Every entry point is called with valid
// arguments (checked: status FA_OK and the launch arguments the layer derived) and with the
// rejected cases (checked: the status, and that nothing was launched).  Exit code 0 and the
// line "api_sanitize ok" mean every check passed.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fa.h"
#include "../../exact_io_aware_fa2_amd/csrc/fa_kernels.hpp"

namespace stub {
extern fa::FwdArgs fwd;
extern fa::BwdArgs bwd;
extern fa::DecodeArgs dec;
extern int calls_fwd_bf16, calls_fwd_fp32, calls_fwd_fp8, calls_bwd, calls_decode;
}  // namespace stub

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, fa_last_error()); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static int launches() {
  return stub::calls_fwd_bf16 + stub::calls_fwd_fp32 + stub::calls_fwd_fp8 + stub::calls_bwd +
         stub::calls_decode;
}

int main() {
  alignas(256) static char mem[1 << 16];
  void* A = mem;
  float* F = reinterpret_cast<float*>(mem);
  const int* I = reinterpret_cast<const int*>(mem);
  const float log2e = 1.4426950408889634f;

  // forward: valid call, then the derived launch arguments
  CHECK(fa_fwd(A, A, A, A, F, 2, 8, 2, 300, 128, 1, 64, -0.25f, nullptr) == FA_OK);
  CHECK(stub::calls_fwd_bf16 == 1);
  CHECK(stub::fwd.B == 2 && stub::fwd.Hq == 8 && stub::fwd.Hkv == 2 && stub::fwd.N == 300);
  CHECK(stub::fwd.d == 128 && stub::fwd.causal == 1 && stub::fwd.window == 64);
  CHECK(fabsf(stub::fwd.c_log2 - 0.25f * log2e) < 1e-7f && stub::fwd.neg_q == 1);
  CHECK(stub::fwd.slopes == nullptr && stub::fwd.cu == nullptr);
  CHECK(fa_fwd(A, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, 0.f, nullptr) == FA_OK);
  CHECK(stub::fwd.c_log2 > 0.f && stub::fwd.neg_q == 0);  // scale 0: tiny positive factor
  CHECK(fa_fwd_alibi(A, A, A, A, F, 1, 4, 4, 16, 64, 1, 0, 0.125f, F + 4, nullptr) == FA_OK);
  CHECK(stub::fwd.slopes == F + 4);
  CHECK(fa_fwd_fp32((float*)A, F, F, F, F, 1, 2, 2, 16, 64, 0, 0, 0.125f, nullptr) == FA_OK);
  CHECK(stub::calls_fwd_fp32 == 1);
  CHECK(fa_fwd_fp8(A, A, A, A, F, 0.5f, 0.25f, 2.f, 1, 2, 2, 16, 128, 1, 0, 0.1f, nullptr) ==
        FA_OK);
  CHECK(stub::calls_fwd_fp8 == 1 && stub::fwd.o_scale == 2.f);
  CHECK(fabsf(stub::fwd.c_log2 - 0.1f * 0.5f * 0.25f * log2e) < 1e-7f);

  // backward: workspace pointer becomes D, the bias pointer passes through
  const size_t need = fa_bwd_workspace_size(2, 8, 2, 300, 128, 1, 0);
  CHECK(need == (2 * 8 * 300 * 4 + 255) / 256 * 256);
  CHECK(fa_bwd(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, A, need, nullptr) ==
        FA_OK);
  CHECK(stub::calls_bwd == 1 && stub::bwd.dvec == F && stub::bwd.slopes == nullptr);
  CHECK(fabsf(stub::bwd.scale - 0.1f) == 0.f && stub::bwd.N == 300);
  CHECK(fa_bwd_alibi(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, A, need, F,
                     nullptr) == FA_OK);
  CHECK(stub::calls_bwd == 2 && stub::bwd.slopes == F);

  // no-allocation backward: the static workspace stands in for the caller's
  CHECK(fa_bwd_noalloc(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, nullptr) ==
        FA_OK);
  CHECK(stub::calls_bwd == 3 && stub::bwd.dvec != nullptr && stub::bwd.dvec != F);
  CHECK(stub::bwd.slopes == nullptr && stub::bwd.N == 300);
  CHECK(fa_bwd_noalloc(A, A, A, A, A, F, A, A, A, 1, 64, 8, 65536, 128, 1, 0, 0.1f, nullptr) ==
        FA_OK);  // 2^22 rows: exactly the limit

  // packed sequences
  CHECK(fa_fwd_varlen(A, A, A, A, F, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, nullptr) == FA_OK);
  CHECK(stub::fwd.cu == I && stub::fwd.ntot == 64 && stub::fwd.N == 40 && stub::fwd.B == 3);
  CHECK(fa_fwd_varlen_alibi(A, A, A, A, F, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, F, nullptr) ==
        FA_OK);
  const size_t vneed = fa_bwd_varlen_workspace_size(64, 4, 2, 128);
  CHECK(fa_bwd_varlen(A, A, A, A, A, F, A, A, A, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, A, vneed,
                      nullptr) == FA_OK);
  CHECK(stub::bwd.cu == I && stub::bwd.ntot == 64);
  CHECK(fa_bwd_varlen_alibi(A, A, A, A, A, F, A, A, A, I, 3, 64, 40, 4, 2, 128, 1, 0, 0.1f, A,
                            vneed, F, nullptr) == FA_OK);

  // decoding: the split count and the workspace split into partial O and LSE
  const int S = fa_decode_num_splits(2, 8, 2, 1, 4096, 128, 4);
  const size_t dneed = fa_decode_workspace_size(2, 8, 2, 1, 4096, 128, 4);
  CHECK(S == 4 && dneed <= sizeof(mem));
  CHECK(fa_decode(A, A, A, I, A, F, 2, 8, 2, 1, 4096, 128, 1, 0, 0.1f, 4, A, dneed, nullptr) ==
        FA_OK);
  CHECK(stub::dec.S == 4 && stub::dec.opart == F && stub::dec.lpart != nullptr);
  CHECK((char*)stub::dec.lpart - (char*)stub::dec.opart >= 4 * 2 * 8 * 1 * 128 * 4);

  // the timing hook is consumed by the next backward call
  CHECK(fa_bwd_time_main_kernel(A, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_bwd_time_main_kernel(A, F) == FA_OK);
  CHECK(fa_bwd(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, A, need, nullptr) ==
        FA_OK);
  CHECK(stub::bwd.ev_start == (hipEvent_t)A && stub::bwd.ev_stop == (hipEvent_t)F);
  CHECK(fa_bwd(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, A, need, nullptr) ==
        FA_OK);
  CHECK(stub::bwd.ev_start == nullptr && stub::bwd.ev_stop == nullptr);

  // rejected calls launch nothing
  const int before = launches();
  CHECK(fa_fwd(nullptr, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, 0.1f, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_fwd(A, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, NAN, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_fwd(A, A, A, A, F, 1, 2, 2, 16, 80, 0, 0, 0.1f, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_fwd(A, A, A, A, F, 1 << 12, 16, 16, 1 << 12, 128, 0, 0, 0.1f, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_fwd(A, A, A, A, F, 0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 256, 0, 0, 0.1f,
               nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_fwd_alibi(A, A, A, A, F, 1, 2, 2, 16, 64, 0, 0, 0.1f, nullptr, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_bwd_noalloc(A, A, A, A, A, F, A, A, A, 1, 64, 8, 65537, 64, 1, 0, 0.1f, nullptr) ==
        FA_ERR_WORKSPACE);  // one row past the static workspace
  CHECK(fa_bwd_noalloc(A, A, A, A, nullptr, F, A, A, A, 1, 4, 2, 64, 64, 1, 0, 0.1f,
                       nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_bwd(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, A, need - 1,
               nullptr) == FA_ERR_WORKSPACE);
  CHECK(fa_bwd(A, A, A, A, A, F, A, A, A, 2, 8, 2, 300, 128, 1, 0, 0.1f, (char*)A + 128, need,
               nullptr) == FA_ERR_WORKSPACE);
  CHECK(fa_bwd_workspace_size(0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 128, 0, 0) == 0);
  CHECK(fa_fwd_varlen(A, A, A, A, F, I, 0x7fffffff, 0x7fffffff, 0x7fffffff, 64, 64, 128, 1, 0,
                      0.1f, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_bwd_varlen_workspace_size(0x7fffffff, 0x7fffffff, 1, 128) == 0);
  CHECK(fa_decode(A, A, A, I, A, F, 0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 0x7fffffff, 128, 1,
                  0, 0.1f, 256, A, 1, nullptr) != FA_OK);
  CHECK(fa_decode_num_splits(0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 0x7fffffff, 128, 0) >= 0);
  CHECK(fa_decode_workspace_size(0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 0x7fffffff, 128, 256)
        >= 0);
  CHECK(fa_fwd_fp8(A, A, A, A, F, 1e30f, 1e30f, 1.f, 1, 2, 2, 16, 64, 0, 0, 1.f, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(launches() == before);
  CHECK(strlen(fa_last_error()) < 512);

  if (failures) {
    printf("api_sanitize: %d failure(s)\n", failures);
    return 1;
  }
  printf("api_sanitize ok\n");
  return 0;
}
