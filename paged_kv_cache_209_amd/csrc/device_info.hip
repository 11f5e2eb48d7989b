// Device queries used to size persistent-style grids. Results are cached per
// (kernel, device); the cache is filled under a mutex, so concurrent first
// calls are safe.
#include <mutex>

#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kFallbackComputeUnits = 256;  // MI355X
constexpr int kCacheSlots = 64;

struct Entry {
  const void* kernel;
  int device;
  int per_cu;
  int cus;
};

std::mutex g_mu;
Entry g_cache[kCacheSlots];
int g_used = 0;

}  // namespace

int resident_workgroups(const void* kernel, int threads, int64_t max_units, int max_per_cu, int* compute_units) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  int per_cu = 0, cus = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    for (int i = 0; i < g_used; ++i) {
      if (g_cache[i].kernel == kernel && g_cache[i].device == device) {
        per_cu = g_cache[i].per_cu;
        cus = g_cache[i].cus;
        break;
      }
    }
    if (cus == 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
        cus = kFallbackComputeUnits;
      (void)hipGetLastError();
      if (g_used < kCacheSlots) g_cache[g_used++] = Entry{kernel, device, per_cu, cus};
    }
  }
  if (max_per_cu > 0 && per_cu > max_per_cu) per_cu = max_per_cu;
  if (compute_units != nullptr) *compute_units = cus;
  int64_t wgs = static_cast<int64_t>(per_cu) * cus;
  if (max_units > 0 && wgs > max_units) wgs = max_units;
  return static_cast<int>(wgs < 1 ? 1 : wgs);
}

}  // namespace pa
