// Host-side helpers of the library: status strings and cached device facts.
#include <atomic>
#include <functional>
#include <mutex>
#include <unordered_map>

#include "launch.hpp"

namespace moe {

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    // zero until first queried; threads that race on the first query all
    // store the same value (relaxed atomics: no data race)
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int resident_blocks_impl(const void* kernel, int block, size_t lds) {
    struct Key {
        const void* k;
        int block;
        size_t lds;
        int dev;
        bool operator==(const Key& o) const { return k == o.k && block == o.block && lds == o.lds && dev == o.dev; }
    };
    struct Hash {
        size_t operator()(const Key& x) const {
            return std::hash<const void*>()(x.k) ^ (std::hash<size_t>()(x.lds) * 31u) ^
                   (static_cast<size_t>(x.block) << 20) ^ (static_cast<size_t>(x.dev) << 40);
        }
    };
    static std::mutex mu;
    static std::unordered_map<Key, int, Hash> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const Key key{kernel, block, lds, dev};
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, lds) != hipSuccess || n < 1) n = 1;
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = n;
    return n;
}

}  // namespace moe

extern "C" const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL_ARG: return "a required pointer is NULL";
        case MOE_ERR_BAD_SHAPE: return "a size is outside the supported range";
        case MOE_ERR_BAD_DTYPE: return "unknown dtype code";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_BAD_ARG: return "a scalar argument is out of range";
        case MOE_ERR_HIP: return "the HIP runtime rejected a launch";
        case MOE_ERR_ALIGN: return "an array pointer is not 16-byte aligned";
        default: return "unknown status";
    }
}
