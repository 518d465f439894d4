// Kernel launchers for the host-only sanitizer build of the library's host code: the
// real ones live with the device code; here every launch reports failure, so the host
// paths run to their end without a device.
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "plan.h"

namespace mhg {
hipError_t launch_fma(int, const LaunchArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma(int, const LaunchArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_fill(const LaunchArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_w8(const LaunchArgs &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_skinny(const LaunchArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mfma32(const LaunchArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_zero_words(void *, int64_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_transpose(const void *, void *, int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_clock_probe(uint64_t *, uint64_t, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace mhg
