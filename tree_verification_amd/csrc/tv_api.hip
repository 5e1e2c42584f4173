// Shared host-side pieces of libtreeverify: device queries and status names.

#include "tv_common.h"

#include <mutex>

namespace {
constexpr int kMaxDevices = 64;
int g_cu[kMaxDevices];
std::once_flag g_once[kMaxDevices];
}  // namespace

int tv_device_cu_count(int* cu_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TV_ERR_HIP;
  std::call_once(g_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_cu[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess) ? prop.multiProcessorCount : 0;
  });
  if (g_cu[dev] <= 0) return TV_ERR_HIP;
  *cu_out = g_cu[dev];
  return TV_OK;
}

extern "C" const char* tv_status_string(int code) {
  switch (code) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID_ARG: return "TV_ERR_INVALID_ARG";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE";
    case TV_ERR_HIP: return "TV_ERR_HIP";
    default: return "unknown status";
  }
}
