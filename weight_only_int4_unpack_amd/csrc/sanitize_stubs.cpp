// Host-only stand-ins for the device side, linked only into the sanitizer
// build of the host code (w4a16_host.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer, run on a machine without a GPU). The argument
// checks, the selector and the pack utilities run for real; every path that
// would launch a kernel stops earlier at the device check on such a
// machine, and these return an error if one is ever reached.
#include <hip/hip_runtime.h>

#include "w4a16_internal.h"

namespace w4a16 {
hipError_t launch_decode(const DecodeParams&, int, bool, int, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill(const PrefillParams&, int, bool, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_prefill_reduce(const PrefillReduceParams&, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_asum(const AsumParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kpacked(const KPackedParams&, int, bool, bool, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_dequant(const DequantParams&, int, bool, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t static_scratch(hipStream_t, void**) { return hipErrorNoDevice; }
}  // namespace w4a16
