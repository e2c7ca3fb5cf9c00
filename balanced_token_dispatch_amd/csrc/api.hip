// Library-wide helpers: status strings and the per-device property cache.
#include <mutex>

#include "common.hpp"

namespace moe {

namespace {
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_once[kMaxDevices];
}  // namespace

// Compute units of the current device (cached per device).
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

}  // namespace moe

extern "C" const char *moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, shape, dtype or op)";
    case MOE_ENOSPACE: return "workspace smaller than the size query (or, for a no-allocation call, than the call needs of its static scratch)";
    case MOE_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}
