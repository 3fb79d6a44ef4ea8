// One-time, per-device set-up of the host side of the library: kernel
// attributes, occupancy queries and device-symbol addresses.  Each value is
// computed once for each device (with that device current) and kept until
// the process ends; concurrent first calls from several threads are safe.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

namespace dsaidx {

constexpr int kMaxDevices = 64;

template <typename T>
class PerDevice {
public:
    // Returns in *out the value f(dev, &value) computed for the current
    // device, running f only on the first call for that device.  A failed
    // f is not cached: the next call runs it again.
    template <typename F>
    hipError_t get(F&& f, T* out) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (!ready_[dev].load(std::memory_order_acquire)) {
            std::lock_guard<std::mutex> g(mu_);
            if (!ready_[dev].load(std::memory_order_relaxed)) {
                T v{};
                e = f(dev, &v);
                if (e != hipSuccess) return e;
                val_[dev] = v;
                ready_[dev].store(true, std::memory_order_release);
            }
        }
        *out = val_[dev];
        return hipSuccess;
    }

private:
    std::mutex mu_;
    std::atomic<bool> ready_[kMaxDevices] = {};
    T val_[kMaxDevices] = {};
};

// Raises a kernel's dynamic-LDS limit to `bytes`, once per device.
inline hipError_t set_lds_limit(PerDevice<int>& once, const void* kernel, int bytes) {
    int done = 0;
    return once.get(
        [&](int, int* v) {
            const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
            *v = 1;
            return e;
        },
        &done);
}

}  // namespace dsaidx
