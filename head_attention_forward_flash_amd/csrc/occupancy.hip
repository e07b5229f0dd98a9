// How many workgroups of a kernel the current device holds at once, queried from the runtime
// once per (device, kernel, block size) and cached.

#include <mutex>
#include <vector>

#include "kernels.h"

namespace mha {

namespace {

struct Resident {
    int device;
    const void* kernel;
    int threads;
    int groups;
};

std::mutex g_lock;
std::vector<Resident> g_cache;

}  // namespace

hipError_t resident_groups(const void* kernel, int threads, int* groups) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> g(g_lock);
        for (const Resident& r : g_cache) {
            if (r.device == dev && r.kernel == kernel && r.threads == threads) {
                *groups = r.groups;
                return hipSuccess;
            }
        }
    }
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess) return e;
    const int n = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    std::lock_guard<std::mutex> g(g_lock);
    g_cache.push_back(Resident{dev, kernel, threads, n});
    *groups = n;
    return hipSuccess;
}

}  // namespace mha
