// tv_device.hip -- per-device facts the launchers need: the compute-unit count
// that sizes the attention plan, and a once-per-(device, kernel) raise of the
// dynamic-LDS limit. Both are cached per device under one mutex (the library
// may be called from several host threads and on several devices).
#include <mutex>
#include <utility>
#include <vector>

#include "tv_launch.h"

namespace tv {
namespace {

std::mutex g_mu;
std::vector<int> g_cus;                                    // per device, 0 = not read yet
std::vector<std::pair<int, const void*>> g_lds_raised;     // (device, kernel) pairs done

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  std::lock_guard<std::mutex> lk(g_mu);
  if ((size_t)dev >= g_cus.size()) g_cus.resize(dev + 1, 0);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return 0;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

hipError_t raise_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  for (const auto& d : g_lds_raised)
    if (d.first == dev && d.second == kernel) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  g_lds_raised.emplace_back(dev, kernel);
  return hipSuccess;
}

}  // namespace tv
