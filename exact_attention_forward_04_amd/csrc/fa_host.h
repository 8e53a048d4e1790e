// fa_host.h -- host-side helpers shared by the library's entry points:
// the per-device check that a gfx950 is current (with its CU count), the
// pointer alignment test and the dynamic-LDS opt-in of a kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>

#include "fa.h"

namespace {

struct DeviceInfo {
  int ok = 0;
  int cus = 0;
  int clock_khz = 0;  // peak shader clock
};

DeviceInfo g_dev[64];
std::once_flag g_dev_once[64];

int current_device(DeviceInfo **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_NO_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return;
    if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return;
    g_dev[dev].cus = p.multiProcessorCount;
    g_dev[dev].clock_khz = p.clockRate;
    g_dev[dev].ok = 1;
  });
  if (!g_dev[dev].ok) return FA_ERR_NO_DEVICE;
  *out = &g_dev[dev];
  return FA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// FA_LOG set to anything but "" or "0" in the environment: one line on
// stderr per kernel launch, naming the kernel variant, its grid, its LDS
// bytes and what the launch covers.  Read once per process.
bool log_on() {
  static const bool on = [] {
    const char *e = std::getenv("FA_LOG");
    return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
  }();
  return on;
}
#define FA_LOG_LAUNCH(...)                        \
  do {                                            \
    if (log_on()) {                               \
      std::fprintf(stderr, "[fa] " __VA_ARGS__);  \
      std::fputc('\n', stderr);                   \
    }                                             \
  } while (0)

// Allow a kernel the dynamic LDS it needs (above the 64 KB default).
template <typename K>
bool allow_lds(K kern, size_t bytes) {
  static std::mutex mu;
  static std::map<const void *, size_t> granted;  // per kernel
  std::lock_guard<std::mutex> lock(mu);
  size_t &g = granted[(const void *)kern];
  if (bytes <= g) return true;
  if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes) != hipSuccess)
    return false;
  g = bytes;
  return true;
}

}  // namespace
