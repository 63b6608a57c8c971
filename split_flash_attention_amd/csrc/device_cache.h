// Per-device caches of launch settings, safe under concurrent calls.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace selattn {

constexpr int kMaxCachedDevices = 64;

// One positive int per device, keyed by a non-negative int (a kernel's LDS size,
// say).  The value is computed by an idempotent function (occupancy queries,
// kernel attributes), so concurrent first calls may both compute it; the slot is
// read and written atomically, and a value is published only after its function
// has returned.  Devices beyond the table, or a failing hipGetDevice, compute
// every time.
class DeviceCache {
public:
    template <typename F>
    int get(int key, F&& compute) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxCachedDevices) return compute();
        const long long want = static_cast<long long>(key) << 32;
        const long long cur = slot_[dev].load(std::memory_order_acquire);
        if (cur != 0 && (cur & ~0xffffffffLL) == want) return static_cast<int>(cur & 0xffffffffLL);
        const int v = compute();
        if (v > 0) slot_[dev].store(want | static_cast<unsigned>(v), std::memory_order_release);
        return v;
    }

private:
    std::atomic<long long> slot_[kMaxCachedDevices];
};

}  // namespace selattn
