// Host-side device queries shared by the launchers.
#include <atomic>

#include "moe_internal.h"

namespace bitffn {

int device_cus() {
  // compute units of each device, asked once per device and kept until the
  // process ends (devices beyond the table are asked every time)
  static std::atomic<int> cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipDeviceProp_t prop;
  const int c = hipGetDeviceProperties(&prop, dev) == hipSuccess ? prop.multiProcessorCount : 256;
  if (dev >= 0 && dev < kMaxDevices) cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

}  // namespace bitffn
