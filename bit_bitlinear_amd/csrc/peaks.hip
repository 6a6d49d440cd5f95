// peaks.hip -- probe kernels that measure the ceilings of one gfx950 GPU: a
// streaming 16-byte copy (HBM) and loops of dense matrix-core instructions
// (i8, FP6 x FP4, bf16) on register operands.  The benchmark times them and
// reports its own kernels against the measured figures beside the published
// peaks.  Not part of the H-BitLinear layer.
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
