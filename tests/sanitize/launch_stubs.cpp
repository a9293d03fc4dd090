// Stand-ins for the kernel launchers of the HIP library, for a host-only build of the ABI layer
// (qv_abi.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.  Each stub counts its calls
// and reports a launch failure, so a test can tell whether a call got past the argument checks.
#include "qv_internal.h"

static int g_launches = 0;

extern "C" int qv_stub_launches(void) { return g_launches; }
extern "C" void qv_stub_reset(void) { g_launches = 0; }

namespace qv {

static hipError_t stub() {
  ++g_launches;
  return hipErrorInvalidValue;
}

hipError_t launch_rotate_quant(const void*, bool, int64_t, int64_t, int64_t, const float*, uint8_t*, float*, int,
                               hipStream_t) {
  return stub();
}
hipError_t launch_w4a4_gemm(const uint8_t*, const float*, const uint8_t*, const float*, const float*, int64_t, int64_t,
                            int64_t, bool, void*, bool, int64_t, hipStream_t) {
  return stub();
}
hipError_t launch_rotate_quant_grouped(const void*, bool, int64_t, int64_t, int64_t, const float*, int64_t, uint8_t*,
                                       float*, hipStream_t) {
  return stub();
}
hipError_t launch_w4a4_gemm_grouped(const uint8_t*, const float*, const uint8_t*, const float*, const float*, int64_t,
                                    int64_t, int64_t, int64_t, bool, void*, bool, int64_t, hipStream_t) {
  return stub();
}
hipError_t launch_w8a8_gemm(const int8_t*, const float*, const int8_t*, const float*, const float*, int64_t, int64_t,
                            int64_t, bool, void*, bool, int64_t, hipStream_t) {
  return stub();
}
hipError_t launch_smooth_calibrate(const void*, bool, int64_t, int64_t, const void*, bool, int64_t, int64_t, int64_t,
                                   float, float*, float*, hipStream_t) {
  return stub();
}

hipError_t noalloc_scratch(void**, size_t*) { return stub(); }
hipError_t launch_w4a4_gemm_requant(const uint8_t*, const float*, const uint8_t*, const float*, const float*, int64_t,
                                    int64_t, int64_t, bool, void*, int64_t, const float*, uint8_t*, float*, unsigned*,
                                    hipStream_t) {
  return stub();
}

}  // namespace qv
