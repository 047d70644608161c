// Host-side helpers of the fp8bs C ABI: argument checks, the gfx950 device
// check (cached per device), launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "fp8bs.h"

namespace fp8bs {

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

struct DeviceInfo {
  int status;      // FP8BS_OK or FP8BS_ERR_DEVICE
  int num_cus;     // compute units
};

// Checks that the current device is a gfx950 and returns its CU count. The
// answer is cached per device id (first call per device queries the runtime).
inline DeviceInfo current_device() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];   // 0 unknown, >0 CU count, -1 not gfx950
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return {FP8BS_ERR_DEVICE, 0};
  }
  if (dev < kMaxDev) {
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return {FP8BS_OK, c};
    if (c < 0) return {FP8BS_ERR_DEVICE, 0};
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return {FP8BS_ERR_DEVICE, 0};
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  const int cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  if (dev < kMaxDev) cached[dev].store(ok ? cus : -1, std::memory_order_relaxed);
  return {ok ? FP8BS_OK : FP8BS_ERR_DEVICE, cus};
}

// Status after a kernel launch.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? FP8BS_OK : FP8BS_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace fp8bs
