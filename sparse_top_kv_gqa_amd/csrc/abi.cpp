// Library-wide parts of the C ABI: error text, version, device property cache.
#include <mutex>
#include <string>
#include <vector>

#include "spk_internal.h"

namespace spk {

namespace {
thread_local std::string g_last_error;
}

spk_status set_error(spk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

int num_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace spk

extern "C" {

SPK_API const char* spk_last_error(void) { return spk::g_last_error.c_str(); }

SPK_API int spk_version(void) { return SPK_VERSION; }

}  // extern "C"
