// splash_clock_probe / splash_realtime_khz: the shader clock over a run of
// kernels, for the benchmark's peak at the measured clock.  Not part of the
// attention computation.  See include/splash.h for the contract.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "errors.h"
#include "splash.h"

namespace {

// s_getreg operands: HW_REG_XCC_ID (hardware register 20 on gfx940 and
// later), bits 3:0 = the XCD; HW_REG_HW_ID (register 4), bits 15:8 = the
// CU, shader array and shader engine inside it.
constexpr int kXccIdReg = (3 << 11) | 20;
constexpr int kHwIdReg = (31 << 11) | 4;

// One wave per work-group: the core-clock cycle counter, the constant-rate
// real-time counter and where the wave runs, read back to back and stored by
// lane 0.  The cycle counters of different CUs are not in step, so only
// stamps taken on the same CU (same location word) can be subtracted.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* out) {
  const uint64_t cycles = __builtin_amdgcn_s_memtime();
  const uint64_t real = __builtin_amdgcn_s_memrealtime();
  const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg(kXccIdReg) & 15u;
  const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg(kHwIdReg) & 0xff00u;
  if (threadIdx.x == 0) {
    uint64_t* o = out + 3 * (size_t)blockIdx.x;
    o[0] = cycles;
    o[1] = real;
    o[2] = (xcc << 16) | hw;
  }
}

}  // namespace

extern "C" int splash_clock_probe(uint64_t* out, int n_groups, void* stream) {
  splash::clear_error();
  if (!out) return splash::fail(SPLASH_EINVAL, "splash_clock_probe: NULL out");
  if (n_groups < 1 || n_groups > 4096)
    return splash::fail(SPLASH_EINVAL, "splash_clock_probe: n_groups %d outside 1..4096", n_groups);
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)n_groups), dim3(64), 0,
                     static_cast<hipStream_t>(stream), out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return splash::fail(SPLASH_EHIP, "splash_clock_probe: launch failed: %s", hipGetErrorString(e));
  return SPLASH_OK;
}

extern "C" int splash_realtime_khz(int* khz) {
  splash::clear_error();
  if (!khz) return splash::fail(SPLASH_EINVAL, "splash_realtime_khz: NULL khz");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return splash::fail(SPLASH_EHIP, "splash_realtime_khz: %s", hipGetErrorString(e));
  return SPLASH_OK;
}
