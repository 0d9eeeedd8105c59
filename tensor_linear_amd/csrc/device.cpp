// Device queries shared by the launchers (kept apart from the argument
// checks in tplinear.cpp, whose host code is also built without the HIP
// runtime for the sanitizer tests).
#include <hip/hip_runtime.h>

#include <atomic>

#include "kernels.h"

namespace tpl {

namespace {
constexpr int MAX_DEVICES = 64;   // devices with an id below this are cached
}

int device_cu_count() {
    static std::atomic<int> cache[MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < MAX_DEVICES) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    if (dev >= 0 && dev < MAX_DEVICES) cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace tpl
