// Device queries shared by the C-ABI source files of libfa.so.
#pragma once

#include <hip/hip_runtime.h>

namespace fa_api {

// Compute units of the current device, cached per device; 0 if the query fails.
inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

}  // namespace fa_api
