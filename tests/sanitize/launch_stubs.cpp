// Host-only stand-ins for the kernel launchers, so that the C ABI and the
// zigzag plan can be built with AddressSanitizer / UndefinedBehaviorSanitizer
// and exercised on the CPU.  Every launcher reports "not supported"; the
// tests that run against this build only reach paths that return before any
// launch (argument validation, empty calls, the host plan).
#include <hip/hip_runtime_api.h>

#include "../../branch_aware_causal_amd/csrc/launch.hpp"

extern "C" const char* hipGetErrorString(hipError_t) { return "launch stubbed in the host-only build"; }
extern "C" hipError_t hipGetLastError() { return hipSuccess; }

namespace bac {
hipError_t launch_main_fwd_valu(const MainArgs&) { return hipErrorNotSupported; }
hipError_t launch_main_bwd_valu(const MainArgs&, int) { return hipErrorNotSupported; }
hipError_t launch_main_fwd_mfma(const MainArgs&) { return hipErrorNotSupported; }
hipError_t launch_main_bwd_mfma(const MainArgs&, int) { return hipErrorNotSupported; }
hipError_t launch_branch_fwd(const BranchArgs&) { return hipErrorNotSupported; }
hipError_t launch_branch_bwd(const BranchArgs&) { return hipErrorNotSupported; }
hipError_t launch_lse_merge(float*, float*, const float*, const float*, int, int, int, int, void*,
                            hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_delta(const void*, int, const void*, int, int, int, int, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_check_index(const int32_t*, const int32_t*, int, int, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_tap_send(void*, uint64_t*, int, const void*, int64_t, uint64_t, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_tap_recv(const void*, const uint64_t*, int, uint64_t, int64_t, void*, int64_t,
                           int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace bac
