// Measurement aid, not part of the quantizer: the shader clock the GPU runs
// at, read in stream order between other launches.
//
// MI355X lowers its shader clock under sustained load (its power management
// picks the clock for windows of a few hundred microseconds), and the
// attention kernels, half bound by their arithmetic, take longer as it
// drops.  One wave spins on a dependent FMA chain and records the shader
// clock counter (clock64, which ticks at the shader clock) and the
// constant-rate wall clock (wall_clock64) around it; their ratio times the
// wall clock's rate is the shader clock of that moment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.hpp"

namespace kvq {

namespace {

__global__ void __launch_bounds__(64) shader_clock_kernel(uint64_t* out, int iters) {
  const uint64_t t0 = clock64();
  const uint64_t r0 = wall_clock64();
  float x = 1.f + static_cast<float>(threadIdx.x) * 1e-9f;
  for (int i = 0; i < iters; ++i) x = fmaf(x, 1.0000001f, 1e-7f);
  const uint64_t t1 = clock64();
  const uint64_t r1 = wall_clock64();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = r1 - r0;
    // keeps the chain alive; never equal to the sentinel for finite x
    out[2] = x == -1.f ? 1u : 0u;
  }
}

}  // namespace

hipError_t launch_shader_clock(uint64_t* out, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(shader_clock_kernel, dim3(1), dim3(64), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace kvq
