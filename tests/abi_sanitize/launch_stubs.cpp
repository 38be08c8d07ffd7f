// Kernel launchers for a host-only build of the C-ABI layer (nvfp4_abi.cpp)
// under AddressSanitizer and UndefinedBehaviorSanitizer: the argument checks
// and status mapping run as in the real library, and any call that gets past
// them finds no device here.  Used by tests/test_abi_sanitized.py only.
#include "nvfp4_internal.h"

namespace nvfp4 {

hipError_t launch_quantize(const void*, int, int64_t, int64_t, int64_t, float*, bool, uint8_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_amax_observe(const void*, int, int64_t, int64_t, int64_t, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gscale_from_amax(const float*, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_quantize_fp8(const void*, int, int64_t, int64_t, int64_t, const float*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_kv_scale_from_amax(const float*, float*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fuse_rescale(uint8_t*, int64_t, float, float, int64_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_zero_i64(int64_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm(int64_t, int64_t, int64_t, const uint8_t*, const uint8_t*, const float*, const uint8_t*,
                       const uint8_t*, const float*, void*, int, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}

}  // namespace nvfp4
