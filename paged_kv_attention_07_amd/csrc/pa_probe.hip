// Read-bandwidth probe (pa_read_probe): a plain streaming read of a device
// buffer, the achievable-bandwidth reference of the decode kernels.  Its
// loads carry the non-temporal hint, as the decode kernels' K/V loads do.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_common.h"
#include "pa_probe.h"

namespace pa {
namespace {

constexpr int kInFlight = 8;  // 16-byte loads in flight per lane

// Work-group g reads 16-byte vectors [g * per, min((g + 1) * per, n)); in
// each step lane l of wave w loads vectors base + (w * kInFlight + k) * 64 + l
// for k < kInFlight, so each load instruction of a wave covers 1 KiB.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* src, int64_t n,
                                                         int64_t per, uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * per;
  const int64_t end = begin + per < n ? begin + per : n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int64_t kStep = 4 * kInFlight * 64;  // vectors per work-group step
  uint32_t acc = 0;
  int64_t i = begin;
  for (; i + kStep <= end; i += kStep) {
    u32x4_t v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k)
      v[k] = __builtin_nontemporal_load(src + i + (wave * kInFlight + k) * 64 + lane);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (int64_t j = i + threadIdx.x; j < end; j += 256) {
    const u32x4_t v = __builtin_nontemporal_load(src + j);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never taken
}

}  // namespace
}  // namespace pa

extern "C" int pa_read_probe(const void* src, size_t bytes, uint32_t* sink,
                             int32_t waves_per_simd, void* stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return PA_ERR_INVALID_ARG;
  if (waves_per_simd != 1 && waves_per_simd != 2 && waves_per_simd != 4)
    return PA_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return PA_ERR_HIP;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t wgs = (int64_t)cus * waves_per_simd;  // 4 waves per work-group
  const int64_t per = (n + wgs - 1) / wgs;
  hipLaunchKernelGGL(pa::read_probe_kernel, dim3((unsigned)wgs), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pa::u32x4_t*>(src), n,
                     per, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
