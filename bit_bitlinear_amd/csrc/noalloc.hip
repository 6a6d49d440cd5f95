// noalloc.hip -- hbl_forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the forward's workspace (activation codes and per-token
// scales, or the FP6 codes and FP4 weights when they fit) lives in a
// file-scope device array of HBL_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: the first call on a device, with that device current, looks up the
// array's device address with hipGetSymbolAddress and keeps it per device;
// only that address is ever passed to kernels.  The entry point calls no
// allocating routine.  All calls on one GPU share the array, so calls that
// overlap on one GPU (different streams, or host threads on one stream
// without ordering) race; nothing in it has to start at zero (the forward
// writes every workspace byte it later reads).
#include <hip/hip_runtime.h>

#include <atomic>

#include "hbl.h"
#include "hbl_device.h"

static_assert(HBL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[HBL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of `scratch` per device ordinal

// The device address of this device's copy of `scratch` (looked up once per
// device, with that device current), or nullptr with *err set.
void* scratch_address(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch_addr[dev].store(p, std::memory_order_release);  // two first calls store the same address
    return p;
}

}  // namespace

extern "C" hbl_status hbl_forward_noalloc(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                                          const uint8_t* W_packed, const float* alpha, int64_t N,
                                          const hbl_config* cfg, void* Y, int32_t y_dtype, void* stream) {
    // every argument is checked before the first HIP call
    hbl_status st = hbl::check_forward_args(X, x_dtype, M, K, gain, W_packed, alpha, N, cfg, Y, y_dtype);
    if (st != HBL_OK || M == 0) return st;
    size_t need = 0;
    if ((st = hbl_workspace_bytes(M, K, cfg, &need)) != HBL_OK) return st;
    if (need > (size_t)HBL_NOALLOC_SCRATCH_BYTES) return HBL_ERR_WORKSPACE;  // beyond the static scratch
    hipError_t e = hipSuccess;
    void* ws = scratch_address(&e);
    if (!ws) {
        hbl::record_hip_error(e);  // reported by hbl_last_hip_error()
        return HBL_ERR_HIP;
    }
    return hbl_forward(X, x_dtype, M, K, gain, W_packed, alpha, N, cfg, Y, y_dtype, ws,
                       (size_t)HBL_NOALLOC_SCRATCH_BYTES, stream);
}
