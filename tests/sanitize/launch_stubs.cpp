// launch_stubs.cpp -- stand-ins for the kernel launchers, for a host-only build of the
// validation layer (fa_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.
// The ABI tests that run against that build pass only argument blocks that validation
// must reject, so reaching any launcher is itself a failure: each stub aborts.
#include <cstdio>
#include <cstdlib>

#include "fa_internal.h"

namespace fa {

[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "launch stub reached: %s (validation let an argument block through)\n", what);
  std::abort();
}

hipError_t launch_fwd(const FwdParams&, int, int, int, hipStream_t) { reached("launch_fwd"); }
hipError_t launch_fwd_dropout(const FwdParams&, int, int, hipStream_t) { reached("launch_fwd_dropout"); }
hipError_t launch_fwd_fp8(const FwdParams&, int, hipStream_t) { reached("launch_fwd_fp8"); }
hipError_t launch_quantize_fp8(const QuantParams&, int, hipStream_t) { reached("launch_quantize_fp8"); }
hipError_t launch_bwd(const BwdParams&, int, hipStream_t) { reached("launch_bwd"); }
hipError_t launch_decode(const DecParams&, int, int, hipStream_t) { reached("launch_decode"); }
hipError_t decode_scratch(void**) { reached("decode_scratch"); }

}  // namespace fa
