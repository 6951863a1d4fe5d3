// Small helper kernels of the layer's set-up and of the GEMM plan timing: a scaled copy (the
// SSM decay A * log2(e) formed once per layer), a fill (clearing flags and states with a kernel,
// so that a captured graph holds no memset node), and a bounded wait on the wall clock.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

__global__ void scale_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n,
                                  float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i] * scale;
}

__global__ void fill_kernel(float* __restrict__ dst, int64_t n, float value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

// One thread waits until the constant-rate wall clock has advanced by `ticks`.  Each pass sleeps
// 32 x 64 clocks (over 0.5 us at any shader clock of this chip), so `max_passes` also ends the
// wait should the counter ever stand still.
__global__ void spin_kernel(int64_t ticks, int64_t max_passes) {
  if (threadIdx.x != 0) return;
  const int64_t t0 = wall_clock64();
  for (int64_t i = 0; i < max_passes && wall_clock64() - t0 < ticks; ++i) __builtin_amdgcn_s_sleep(32);
}

}  // namespace

hipError_t launch_scale_copy(const float* src, float* dst, int64_t n, float scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_copy_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                     src, dst, n, scale);
  return hipGetLastError();
}

hipError_t launch_fill(float* dst, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

hipError_t launch_spin(int microseconds, hipStream_t s) {
  if (microseconds <= 0) return hipSuccess;
  int rate_khz = 0;   // wall-clock ticks per millisecond
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate_khz <= 0)
    rate_khz = 100000;   // gfx9's 100 MHz
  const int64_t ticks = static_cast<int64_t>(microseconds) * rate_khz / 1000;
  // below 8 GHz a microsecond holds fewer than 4 passes, so the cap never ends a wait early
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, s, ticks, static_cast<int64_t>(microseconds) * 4 + 16);
  return hipGetLastError();
}

}  // namespace hymba
