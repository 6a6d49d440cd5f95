// peaks.hip -- probe kernels that measure the ceilings of one gfx950 GPU: a
// streaming 16-byte copy (HBM), loops of dense matrix-core instructions
// (i8, FP6 x FP4, bf16) on register operands, and the data path of one
// compute unit (LDS reads, LDS-direct loads, and the two mixed with
// matrix-core work in the proportions of one FP6 x FP4 GEMM K step).  The
// benchmark times them and reports its own kernels against the measured
// figures beside the published peaks.  Not part of the H-BitLinear layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hbl_peaks.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kCopyThreads = 256, kCopyUnroll = 4;

// Each thread copies kCopyUnroll 16-byte vectors spaced one block apart,
// issuing all loads before the stores.
__global__ __launch_bounds__(kCopyThreads) void peak_copy_kernel(const uint4* __restrict__ src,
                                                                uint4* __restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < n) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < n) dst[i] = v[u];
    }
}

// Streaming read: each thread loads kCopyUnroll 16-byte vectors spaced one
// block apart and folds them into one word, which it stores only if it equals
// a value the data never produces (so the loads cannot be dropped and the
// kernel writes nothing).
__global__ __launch_bounds__(kCopyThreads) void peak_read_kernel(const uint4* __restrict__ src, int64_t n,
                                                                uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        v[u] = i < n ? src[i] : make_uint4(0, 0, 0, 0);
    }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (x == 0x9E3779B9u) sink[(int64_t)blockIdx.x * kCopyThreads + threadIdx.x] = x;
}

// Streaming write: each thread stores kCopyUnroll 16-byte vectors spaced one
// block apart; nothing is read.
__global__ __launch_bounds__(kCopyThreads) void peak_write_kernel(uint4* __restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
    const uint4 v = make_uint4((uint32_t)base, (uint32_t)blockIdx.x, 0x5A5A5A5Au, 0u);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = base + (int64_t)u * kCopyThreads;
        if (i < n) dst[i] = v;
    }
}

// An empty kernel: the per-launch floor of a grid of the given size.
__global__ __launch_bounds__(256) void peak_empty_kernel() {}

template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(int32_t* __restrict__ out, int iters) {
    const int t = (int)threadIdx.x;
    int32_t res = 0;
    if constexpr (KIND == HBL_PEAK_MFMA_I8) {
        const v4i a = {t, t * 3 + 1, t * 5 + 2, t * 7 + 3};
        const v4i b = {t * 11 + 4, t * 13 + 5, t * 17 + 6, t * 19 + 7};
        v16i acc[4] = {};
        for (int it = 0; it < iters; it++)
#pragma unroll
            for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
            for (int r = 0; r < 16; r++) res += acc[c][r];
    } else if constexpr (KIND == HBL_PEAK_MFMA_F6F4) {
        // FP6 and FP4 have no Inf or NaN encodings: any bits are finite values
        const v8i a = {t, t * 3 + 1, t * 5 + 2, t * 7 + 3, t * 9 + 4, t * 11 + 5, 0, 0};
        const v8i b = {t * 13 + 6, t * 17 + 7, t * 19 + 8, t * 23 + 9, 0, 0, 0, 0};
        v16f acc[4] = {};
        for (int it = 0; it < iters; it++)
#pragma unroll
            for (int c = 0; c < 4; c++)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 3, 4, 0, 0, 0, 0);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
            for (int r = 0; r < 16; r++) s += acc[c][r];
        res = __float_as_int(s);
    } else {
        v8bf a, b;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            a[e] = (__bf16)(0.0078125f * (float)((t + e) & 7));
            b[e] = (__bf16)(-0.0078125f * (float)((t * 3 + e) & 7));
        }
        v16f acc[4] = {};
        for (int it = 0; it < iters; it++)
#pragma unroll
            for (int c = 0; c < 4; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < 4; c++)
#pragma unroll
            for (int r = 0; r < 16; r++) s += acc[c][r];
        res = __float_as_int(s);
    }
    out[(int64_t)blockIdx.x * 256 + t] = res;
}

// ---- data path of one compute unit
constexpr int kLdsThreads = 512;             // 8 waves, two per SIMD
constexpr int kLdsBytes = 96 * 1024;         // > 80 KiB: one workgroup per compute unit
constexpr int kLdsWaveSpan = 10 * 1024;      // LDS-direct ring of a wave: 2 rounds x 5 KiB

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// One LDS-direct load: lane l's 16 bytes at voff of the resource land at LDS
// byte lds_addr + 16*l (M0 holds lds_addr and is restored); no register result.
__device__ __forceinline__ void peak_lds_direct16(v4u desc, uint32_t lds_addr, uint32_t voff) {
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

// s_waitcnt on the vector-memory counter alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void peak_wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int KIND>
__global__ __launch_bounds__(kLdsThreads, 1) void peak_lds_kernel(const uint8_t* __restrict__ src, uint32_t src_mask,
                                                                 int iters, int64_t* __restrict__ clk,
                                                                 uint32_t* __restrict__ sink) {
    constexpr bool kLoads = KIND != HBL_PEAK_LDS_READ && KIND != HBL_PEAK_LDS_KSTEP_NOLOAD;
    constexpr bool kReads = KIND != HBL_PEAK_LDS_DIRECT;
    constexpr bool kMfma = KIND == HBL_PEAK_LDS_KSTEP || KIND == HBL_PEAK_LDS_KSTEP_NOBAR ||
                           KIND == HBL_PEAK_LDS_KSTEP_NOLOAD;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kLdsBytes / 16; i += kLdsThreads)
        reinterpret_cast<uint4*>(lds)[i] = make_uint4(i, 3 * i + 1, 5 * i + 2, 7 * i + 3);
    __syncthreads();
    const uint64_t a = (uint64_t)src;
    const v4u desc = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, src_mask + 1u, 0x00020000u};
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr + (uint32_t)(wave * kLdsWaveSpan));
    const uint32_t first = (uint32_t)((blockIdx.x * 8 + wave) * 5) * 1024u + (uint32_t)lane * 16u;
    auto issue = [&](int it) {
        if constexpr (kLoads) {
#pragma unroll
            for (int u = 0; u < 5; u++)
                peak_lds_direct16(desc, ring + (uint32_t)((it & 1) * 5120 + u * 1024),
                                  (first + (uint32_t)u * 1024u + (uint32_t)it * 40960u) & src_mask);
        }
    };
    long long t0 = 0, r0 = 0;
    if (tid == 0) {
        t0 = (long long)__builtin_amdgcn_s_memtime();
        r0 = (long long)__builtin_amdgcn_s_memrealtime();
    }
    uint4 x = make_uint4(0, 0, 0, 0);
    v16f acc[8] = {};
    v8i fa = {lane, 1, 2, 3, 4, 5, 0, 0};
    const v8i fb = {lane ^ 5, 3, 2, 1, 0, 0, 0, 0};
    issue(0);
    issue(1);
    for (int it = 0; it < iters; it++) {
        if constexpr (kLoads) peak_wait_vmcnt<5>();  // this round's loads have landed
        if constexpr (KIND == HBL_PEAK_LDS_KSTEP || KIND == HBL_PEAK_LDS_KSTEP_NOLOAD)
            asm volatile("s_barrier" ::: "memory");
        issue(it + 2 < iters ? it + 2 : iters - 1);
        if constexpr (kReads) {
            // a wave reads its own ring and the next wave's: offsets below 86 KiB
            const uint8_t* rd = lds + wave * kLdsWaveSpan + lane * 16 + (it & 3) * 64;
            uint4 f[14];
#pragma unroll
            for (int q = 0; q < 14; q++) f[q] = *reinterpret_cast<const uint4*>(rd + q * 1024);
            if constexpr (kMfma) {
#pragma unroll
                for (int m = 0; m < 16; m++) {  // one LDS read between consecutive instructions
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    acc[m & 7] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc[m & 7], 3, 4, 0, 0, 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
#pragma unroll
            for (int q = 0; q < 14; q += 2) {
                x.x ^= f[q].x ^ f[q + 1].x;
                x.y ^= f[q].y ^ f[q + 1].y;
                x.z ^= f[q].z ^ f[q + 1].z;
                x.w ^= f[q].w ^ f[q + 1].w;
            }
            if constexpr (kMfma) fa[0] ^= (int)(x.x & 1u);  // the next round's instructions use this round's reads
        }
    }
    peak_wait_vmcnt<0>();  // no LDS-direct load may be in flight when the workgroup ends
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) s += acc[j][r];
    const uint32_t v = x.x ^ x.y ^ x.z ^ x.w ^ __float_as_uint(s);
    if (v == 0x9E3779B9u) sink[blockIdx.x] = v;
    if (tid == 0) {
        clk[2 * (int64_t)blockIdx.x] = (long long)__builtin_amdgcn_s_memtime() - t0;
        clk[2 * (int64_t)blockIdx.x + 1] = (long long)__builtin_amdgcn_s_memrealtime() - r0;
    }
}

template <int KIND>
int launch_peak_lds(const void* src, uint32_t mask, int blocks, int iters, int64_t* clk, uint32_t* sink,
                    hipStream_t s) {
    auto k = peak_lds_kernel<KIND>;
    if (hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
        return 2;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(kLdsThreads), kLdsBytes, s, (const uint8_t*)src, mask, iters, clk, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int64_t ops_per_instruction(int kind) {
    switch (kind) {
        case HBL_PEAK_MFMA_I8: return 2LL * 32 * 32 * 32;
        case HBL_PEAK_MFMA_F6F4: return 2LL * 32 * 32 * 64;
        case HBL_PEAK_MFMA_BF16: return 2LL * 32 * 32 * 16;
        default: return -1;
    }
}

}  // namespace

extern "C" int hbl_peak_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return 1;
    if (bytes == 0) return 0;
    if (!src || !dst || ((uintptr_t)src | (uintptr_t)dst) % 16) return 1;
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    if (s < d + bytes && d < s + bytes) return 1;
    const int64_t n = bytes / 16;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return 1;
    hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, (hipStream_t)stream,
                       (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int64_t hbl_peak_mfma_ops(int kind, int blocks, int iters) {
    const int64_t per = ops_per_instruction(kind);
    if (per < 0 || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 24)) return -1;
    return per * 4 * 4 * (int64_t)blocks * iters;  // 4 waves per block, 4 instructions per round
}

extern "C" int hbl_peak_mfma(int kind, int32_t* out, int64_t out_len, int blocks, int iters, void* stream) {
    if (hbl_peak_mfma_ops(kind, blocks, iters) < 0 || !out || out_len < (int64_t)blocks * 256) return 1;
    const hipStream_t s = (hipStream_t)stream;
    switch (kind) {
        case HBL_PEAK_MFMA_I8:
            hipLaunchKernelGGL(peak_mfma_kernel<HBL_PEAK_MFMA_I8>, dim3(blocks), dim3(256), 0, s, out, iters);
            break;
        case HBL_PEAK_MFMA_F6F4:
            hipLaunchKernelGGL(peak_mfma_kernel<HBL_PEAK_MFMA_F6F4>, dim3(blocks), dim3(256), 0, s, out, iters);
            break;
        default:
            hipLaunchKernelGGL(peak_mfma_kernel<HBL_PEAK_MFMA_BF16>, dim3(blocks), dim3(256), 0, s, out, iters);
            break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hbl_peak_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_len, void* stream) {
    if (bytes <= 0 || bytes % 16 || !src || !sink || (uintptr_t)src % 16) return 1;
    const int64_t n = bytes / 16;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF || sink_len < blocks * kCopyThreads) return 1;
    hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, (hipStream_t)stream,
                       (const uint4*)src, n, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hbl_peak_write(void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return 1;
    if (bytes == 0) return 0;
    if (!dst || (uintptr_t)dst % 16) return 1;
    const int64_t n = bytes / 16;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    const int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return 1;
    hipLaunchKernelGGL(peak_write_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, (hipStream_t)stream,
                       (uint4*)dst, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int64_t hbl_peak_read_sink_len(int64_t bytes) {
    if (bytes <= 0 || bytes % 16) return -1;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    return (bytes / 16 + per_block - 1) / per_block * kCopyThreads;
}

extern "C" int hbl_peak_empty(int blocks, void* stream) {
    if (blocks < 1 || blocks > (1 << 20)) return 1;
    hipLaunchKernelGGL(peak_empty_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int hbl_peak_lds(int kind, const void* src, int64_t src_bytes, int blocks, int iters, int64_t* clk,
                            int64_t clk_len, uint32_t* sink, int64_t sink_len, void* stream) {
    if (kind < HBL_PEAK_LDS_READ || kind > HBL_PEAK_LDS_KSTEP_NOLOAD) return 1;
    if (blocks < 1 || blocks > (1 << 20) || iters < 2 || iters > (1 << 24)) return 1;
    if (!clk || clk_len < 2 * (int64_t)blocks || !sink || sink_len < blocks) return 1;
    uint32_t mask = 0;
    if (kind != HBL_PEAK_LDS_READ && kind != HBL_PEAK_LDS_KSTEP_NOLOAD) {
        if (!src || (uintptr_t)src % 16) return 1;
        if (src_bytes < (1 << 16) || src_bytes > (1 << 30) || (src_bytes & (src_bytes - 1)) != 0) return 1;
        mask = (uint32_t)(src_bytes - 1);
    }
    const hipStream_t s = (hipStream_t)stream;
    switch (kind) {
        case HBL_PEAK_LDS_READ: return launch_peak_lds<HBL_PEAK_LDS_READ>(src, mask, blocks, iters, clk, sink, s);
        case HBL_PEAK_LDS_DIRECT: return launch_peak_lds<HBL_PEAK_LDS_DIRECT>(src, mask, blocks, iters, clk, sink, s);
        case HBL_PEAK_LDS_KSTEP: return launch_peak_lds<HBL_PEAK_LDS_KSTEP>(src, mask, blocks, iters, clk, sink, s);
        case HBL_PEAK_LDS_KSTEP_NOBAR:
            return launch_peak_lds<HBL_PEAK_LDS_KSTEP_NOBAR>(src, mask, blocks, iters, clk, sink, s);
        default: return launch_peak_lds<HBL_PEAK_LDS_KSTEP_NOLOAD>(src, mask, blocks, iters, clk, sink, s);
    }
}
