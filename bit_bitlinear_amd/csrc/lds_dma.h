// lds_dma.h -- global -> LDS direct loads and the waits around them (gfx950).
// Internal header shared by the GEMM kernels.
#pragma once
#include "hbl_device.h"

namespace hbl {
namespace {

// Buffer stores: an offset outside the resource is dropped by the hardware.
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond every resource: store dropped

// Raw buffer descriptor words (base, stride 0, byte range, format word) as
// four scalar registers; the same resource make_rsrc builds.
HBL_DEVINL v4u rsrc_words(const void* base, int64_t bytes) {
    const uint64_t a = (uint64_t)base;
    const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
    return v4u{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)lim, 0x00020000u};
}

// One LDS-direct load: every lane fetches 16 bytes at voff of the resource and
// the wave's 64 results land contiguously at LDS byte address lds_addr (taken
// from M0, which is restored).  Written as inline asm so that the compiler
// does not treat every later LDS read as dependent on it: the kernel waits
// for these loads itself (wait_vmcnt) before the barrier that publishes them.
// The instruction has no register result.
HBL_DEVINL void lds_dma16(v4u desc, uint32_t lds_addr, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(desc)
        : "memory");
}

// s_waitcnt that waits for the vector-memory counter only (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
HBL_DEVINL void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier with no implied memory wait (the caller has waited for
// what it publishes); the memory clobber keeps LDS accesses on their side.
HBL_DEVINL void barrier_no_wait() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace
}  // namespace hbl
