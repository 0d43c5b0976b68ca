// Shader-clock probe: the clock the compute units actually run at, measured
// on the device.  Each workgroup (one wavefront) runs a dependent chain of
// VALU work until the fixed 100 MHz counter (s_memrealtime) has advanced by
// `ticks`, and stores how far the shader cycle counter (s_memtime) and the
// reference counter advanced; their ratio times 100 MHz is the mean shader
// clock over that span.  Run on its own stream while a benchmark's timed
// launches run on another, one such workgroup measures the clock under the
// benchmark's load while taking one wave slot of the chip.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa2.h"

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* __restrict__ out,
                                                         unsigned long long ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x * 1e-3f, y = 1.0001f;
  unsigned long long r1 = r0;
  // bounded: the reference counter advances at a fixed rate
  while (r1 - r0 < ticks) {
#pragma unroll 1
    for (int i = 0; i < 64; ++i) {
      x = fmaf(x, y, 1e-7f);
      y = fmaf(y, 0.9999f, 1e-4f);
    }
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x + 0] = t1 - t0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = (unsigned long long)__float_as_uint(x + y);  // keeps the chain
  }
}

}  // namespace

extern "C" int fa2_clock_probe(int workgroups, unsigned long long ticks, unsigned long long* out, void* stream) {
  if (out == nullptr || workgroups < 1 || workgroups > 65536) return FA2_ERR_INVALID_ARG;
  if (ticks < 1 || ticks > 1000000000ULL) return FA2_ERR_INVALID_ARG;  // at most 10 s
  if ((reinterpret_cast<uintptr_t>(out) & 7) != 0) return FA2_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)workgroups), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), out, ticks);
  return hipGetLastError() == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}
