// Host-side launch helper: launches with hipLaunchKernel so the launch status
// is returned directly (not read from the thread's sticky last-error slot).
#pragma once

#include <tuple>
#include <utility>

#include "common.hpp"

namespace moe {

template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, void* stream,
           Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
    std::tuple<KArgs...> values(std::forward<Args>(args)...);
    void* ptrs[sizeof...(KArgs)];
    std::apply([&](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, values);
    return hip_status(hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs,
                                      shmem, static_cast<hipStream_t>(stream)));
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Blocks of `block` threads with `lds` bytes of dynamic LDS that fit on one
// CU at once (at least 1); cached per (kernel, block, lds).
int resident_blocks_impl(const void* kernel, int block, size_t lds);

template <typename... KArgs>
int resident_blocks(void (*kernel)(KArgs...), int block, size_t lds) {
    return resident_blocks_impl(reinterpret_cast<const void*>(kernel), block, lds);
}

}  // namespace moe
