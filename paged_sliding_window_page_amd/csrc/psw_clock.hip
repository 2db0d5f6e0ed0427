// Shader clock under matrix-core load.  The MFMA roofline is quoted at the
// part's nominal 2.4 GHz, but with every CU issuing bf16 MFMAs the shader clock
// settles lower; this measures it so a benchmark can also report the fraction
// of the clock-adjusted peak.  Each work-group is eight waves of back-to-back
// independent v_mfma_f32_32x32x16_bf16 (the occupancy and instruction mix of the
// prefill kernels' matrix phases); lane 0 of every work-group reads the shader
// clock counter (s_memtime) and the constant-rate counter (s_memrealtime)
// around the loop.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "psw.h"
#include "psw_device.hpp"
#include "psw_host.hpp"

namespace psw_dev {
namespace {

__global__ __launch_bounds__(512, 1) void mfma_clock_kernel(unsigned long long* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f / (1 + threadIdx.x % 7 + e));
    b[e] = (__bf16)(1.0f / (2 + threadIdx.x % 5 + e));
  }
  f32x16 acc[4] = {};
  __syncthreads();
  const unsigned long long c0 = clock64(), r0 = wall_clock64();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), r1 = wall_clock64();
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += acc[k][threadIdx.x % 16];
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x + 0] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = __float_as_uint(s);  // keeps the MFMAs alive
  }
}

}  // namespace
}  // namespace psw_dev

extern "C" int psw_measure_mfma_clock(psw_stream_t stream, double* mhz) {
  psw::clear_error();
  if (!mhz) return psw::fail(PSW_E_NULL, "mhz is NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1, cus = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      cus <= 0 || wall_khz <= 0)
    return psw::fail(PSW_E_HIP, "device attributes unavailable");
  unsigned long long* d = nullptr;
  const size_t bytes = sizeof(unsigned long long) * 3 * size_t(cus);
  if (hipMalloc(reinterpret_cast<void**>(&d), bytes) != hipSuccess)
    return psw::fail(PSW_E_HIP, "hipMalloc of the clock probe buffer failed");
  std::vector<unsigned long long> h(3 * size_t(cus), 0);
  hipError_t e = hipSuccess;
  // one warm-up launch (clocks ramp under load), then the measured one
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
    hipLaunchKernelGGL(psw_dev::mfma_clock_kernel, dim3(cus), dim3(512), 0, s, d, 20000);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(h.data(), d, bytes, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d);
  if (e != hipSuccess) return psw::fail(PSW_E_HIP, hipGetErrorString(e));
  double cyc = 0.0, ticks = 0.0;
  for (int i = 0; i < cus; ++i) {
    cyc += double(h[3 * i]);
    ticks += double(h[3 * i + 1]);
  }
  if (ticks <= 0.0) return psw::fail(PSW_E_HIP, "clock probe read no time");
  *mhz = cyc / ticks * (wall_khz / 1000.0);
  return PSW_OK;
}
