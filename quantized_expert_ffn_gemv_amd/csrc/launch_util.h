// Host-side sizing of persistent launches.
#pragma once

#include <atomic>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace moe {

// Compute units of the current device (cached on first use).
inline int device_cus() {
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        return n;
    }();
    return cus;
}

// Workgroups of a persistent launch: as many as fit on the chip at once (from
// the kernel's registers and LDS), never more than there can be items, at
// least one.  `cache` (one per kernel, owned by the caller) keeps the
// occupancy answer for the last LDS size.
template <typename K>
inline unsigned persistent_blocks(K kernel, std::atomic<uint64_t>& cache, int block, size_t lds, long max_items) {
    const uint64_t c = cache.load(std::memory_order_relaxed);
    int per_cu = (int)(c & 0xFF);
    if (per_cu == 0 || (c >> 8) != lds) {
        per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds) != hipSuccess || per_cu < 1)
            per_cu = 1;
        per_cu = per_cu > 8 ? 8 : per_cu;
        cache.store(((uint64_t)lds << 8) | (uint64_t)per_cu, std::memory_order_relaxed);
    }
    const long g = (long)per_cu * device_cus();
    const long n = max_items < g ? max_items : g;
    return (unsigned)(n > 0 ? n : 1);
}

}  // namespace moe
