// kernels_probe.hip -- a one-wave clock probe for measurements.  It counts the shader
// clock (s_memtime) over a window of the constant 100 MHz real-time counter
// (s_memrealtime); launched on a second stream beside a run of GEMM calls it reads the
// clock that those calls run at.  It needs no LDS and a handful of registers, so it
// fits on a compute unit next to any GEMM workgroup, and it sleeps between reads of
// the real-time counter so that it takes almost no issue slots from them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhg {
namespace {

// out[0] = shader-clock cycles, out[1] = real-time ticks (>= ticks) of the window.
// The real-time counter advances at a fixed rate, so every wave leaves the loop.
__global__ void __launch_bounds__(64) clock_probe(uint64_t *out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(32);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, uint64_t ticks, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe, dim3(1), dim3(64), 0, s, out, ticks);
  return hipGetLastError();
}

}  // namespace mhg
