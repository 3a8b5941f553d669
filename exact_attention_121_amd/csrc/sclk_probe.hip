// Shader-clock probe and device facts for the benchmark (not part of the
// attention path).
//
// One wave reads the shader-clock cycle counter (clock64) and the
// constant-rate wall counter (wall_clock64, hipDeviceAttributeWallClockRate
// ticks per second) until wall_ticks wall ticks have passed, then writes both
// differences: cycles / seconds is the mean shader clock of the CU it ran on
// over that window.  Launched on a second stream while the timed kernels run,
// it measures the clock under their load.  The loop is bounded by the wall
// counter, so the wave always exits; the results leave through an ordinary
// vector store.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__global__ void sclk_probe_kernel(unsigned long long* out, unsigned long long wall_ticks) {
  if (threadIdx.x != 0) return;
  const unsigned long long w0 = wall_clock64();
  const unsigned long long c0 = clock64();
  unsigned long long w = w0;
  while (w - w0 < wall_ticks) {
    __builtin_amdgcn_s_sleep(8);
    w = wall_clock64();
  }
  const unsigned long long c1 = clock64();
  out[0] = c1 - c0;
  out[1] = w - w0;
}

}  // namespace

// Wall counter rate in kHz (hipDeviceAttributeWallClockRate of the current
// device), or 0 on error.
extern "C" int attn_wall_clock_khz() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  return hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? khz : 0;
}

// out: device pointer to two uint64 (cycles, wall ticks); wall_ticks: length
// of the window in wall ticks (at most 10 s of them); stream: HIP stream or
// NULL.  Returns 0, or 1 on a bad argument or launch error.
extern "C" int attn_sclk_probe(unsigned long long* out, unsigned long long wall_ticks, void* stream) {
  const int khz = attn_wall_clock_khz();
  if (out == nullptr || khz <= 0 || wall_ticks > static_cast<unsigned long long>(khz) * 10000ull) return 1;
  hipLaunchKernelGGL(sclk_probe_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), out, wall_ticks);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Compute units and the maximum shader clock (kHz) of the current device, as
// the runtime reports them (hipDeviceAttributeMultiprocessorCount,
// hipDeviceAttributeClockRate).  Returns 0, or 1 on error.
extern "C" int attn_device_info(int* cus, int* max_clock_khz) {
  int dev = 0;
  if (cus == nullptr || max_clock_khz == nullptr || hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1;
  return hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, dev) == hipSuccess ? 0 : 1;
}
