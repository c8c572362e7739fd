// Host-only stand-ins for the kernel launchers of libfa.so, for the sanitizer build of the
// C ABI layer (tests/test_abi.py): each records the arguments it was given and returns
// hipSuccess without touching a GPU, so the validation and argument marshalling of
// fa_api.hip run under AddressSanitizer / UndefinedBehaviorSanitizer on any host.
#include <string.h>

#include "../../exact_io_aware_fa2_amd/csrc/fa_kernels.hpp"

namespace stub {
fa::FwdArgs fwd;
fa::BwdArgs bwd;
fa::DecodeArgs dec;
int calls_fwd_bf16 = 0, calls_fwd_fp32 = 0, calls_fwd_fp8 = 0, calls_bwd = 0, calls_decode = 0;
}  // namespace stub

namespace fa {
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t) {
  stub::fwd = a;
  ++stub::calls_fwd_bf16;
  return hipSuccess;
}
hipError_t launch_fwd_fp32(const FwdArgs& a, hipStream_t) {
  stub::fwd = a;
  ++stub::calls_fwd_fp32;
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t) {
  stub::fwd = a;
  ++stub::calls_fwd_fp8;
  return hipSuccess;
}
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t) {
  stub::bwd = a;
  ++stub::calls_bwd;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  stub::dec = a;
  ++stub::calls_decode;
  return hipSuccess;
}
hipError_t launch_mfma_probe(float*, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_atomic_probe(float*, int, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_issue_probe(float*, int, int, int, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_fp8_product_probe(const uint8_t*, const uint8_t*, float*, int, hipStream_t) {
  return hipSuccess;
}
// The static workspace of the no-allocation backward: a host address that only flows into the
// recorded arguments.
hipError_t noalloc_scratch(float** ptr) {
  alignas(256) static float fake[64];
  *ptr = fake;
  return hipSuccess;
}
}  // namespace fa
