// lds_attr.h -- host-side helper: raise a kernel's dynamic LDS limit once per
// device.  Internal header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace hbl {

// hipFuncSetAttribute(MaxDynamicSharedMemorySize, bytes) for the current
// device, once per device and kernel: `done` is a per-kernel mask of the
// devices (ordinals 0..31) already set.  Concurrent first calls may both set
// the attribute, which is harmless.
template <typename Kernel>
hipError_t set_dynamic_lds(Kernel kern, size_t bytes, std::atomic<uint32_t>& done) {
    if (bytes == 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint32_t bit = 1u << (dev & 31);
    if (dev < 32 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && dev < 32) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

}  // namespace hbl
