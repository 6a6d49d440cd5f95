// head_quant.hip -- low-bit attention states (gfx950): every (token, head)
// vector of post-RoPE Q, K or V is quantised by its absmax to unsigned b-bit
// integers (b = 3, 4 or 8), with no calibration data.  Follows the 新智元
// "微软 BitNet v2" repost, section "实验结果" (low-bit attention: the QKV heads
// are quantised directly to unsigned integers by absmax; a 3-bit KV cache
// keeps the accuracy of a full-precision one).  The formula is not on the
// pages; the reading: a symmetric absmax quantiser whose signed code is
// stored with the offset 2^(b-1):
//   gamma = max|x|, Qp = 2^(b-1) - 1, s = Qp/(gamma+eps), d = gamma/Qp,
//   u = clamp(rint(x*s), -Qp, Qp) + 2^(b-1)        (gamma = 0: s = d = 0; so too
//   when eps = 0 and Qp/gamma overflows fp32)
//
// HBM-bound streaming kernel.  Lane l of the grid takes the 8 consecutive
// elements 8*(l % G) .. +7 of head vector l / G (G = D/8 lanes per vector,
// 4 to 32, so a vector's lanes are aligned within one wave): one 16-byte load
// for bf16, two for fp32; the G lanes form max|x| with xor shuffles; each
// lane writes its 8 codes as one 8-byte (b = 8), 4-byte (b = 4) or 3-byte
// (b = 3: a 2-byte and a 1-byte store, the vector's bit string has code j at
// bits 3j) piece, and lane 0 of the vector writes d.
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int kHqThreads = 256;

template <typename Tin, int D, int BITS>
__global__ __launch_bounds__(kHqThreads) void head_quant_kernel(const Tin* __restrict__ X, int64_t V, float eps,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ d_out) {
    constexpr int G = D / 8;
    static_assert(G >= 4 && G <= 32 && (G & (G - 1)) == 0, "head vectors of 32 to 256 elements");
    const int64_t gid = (int64_t)blockIdx.x * kHqThreads + threadIdx.x;
    const int64_t v = gid / G;
    const int j = (int)(gid % G);
    const bool live = v < V;
    float x[8];
    if (live) {
        const Tin* p = X + v * D + 8 * j;
        if constexpr (sizeof(Tin) == 4) {
            const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
            const uint4 q = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) x[i] = 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(x[i]));
#pragma unroll
    for (int o = 1; o < G; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));  // every lane of the wave takes part
    if (!live) return;
    constexpr int zp = 1 << (BITS - 1), qp = zp - 1;
    const float gamma = a;
    float s = gamma == 0.f ? 0.f : (float)qp / (gamma + eps);
    // eps = 0 and gamma below qp / FLT_MAX: the multiplier overflows; the
    // vector is taken as gamma = 0 (every code at the zero point)
    const bool zero = gamma == 0.f || __builtin_isinf(s);
    if (zero) s = 0.f;
    if (j == 0) d_out[v] = zero ? 0.f : gamma / (float)qp;
    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; i++) u[i] = (uint32_t)((int)rintf(fminf(fmaxf(x[i] * s, (float)-qp), (float)qp)) + zp);
    if constexpr (BITS == 8) {
        uint2 o;
        o.x = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
        o.y = u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24);
        *reinterpret_cast<uint2*>(codes + v * D + 8 * j) = o;
    } else if constexpr (BITS == 4) {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) o |= u[i] << (4 * i);
        *reinterpret_cast<uint32_t*>(codes + v * (D / 2) + 4 * j) = o;
    } else {
        uint32_t o = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) o |= u[i] << (3 * i);
        // 3 bytes at byte 3j of the vector (3D/8 bytes per vector, an even number,
        // so the piece starts on an even byte exactly when j is even)
        uint8_t* p = codes + v * (3 * D / 8) + 3 * j;
        if ((j & 1) == 0) {
            *reinterpret_cast<uint16_t*>(p) = (uint16_t)o;
            p[2] = (uint8_t)(o >> 16);
        } else {
            p[0] = (uint8_t)o;
            *reinterpret_cast<uint16_t*>(p + 1) = (uint16_t)(o >> 8);
        }
    }
}

template <typename Tin, int D>
hipError_t launch_d(const Tin* X, int64_t V, int bits, float eps, uint8_t* codes, float* d_out, hipStream_t s) {
    const int64_t lanes = V * (D / 8);
    const int64_t blocks = (lanes + kHqThreads - 1) / kHqThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (bits) {
        case 3: hipLaunchKernelGGL((head_quant_kernel<Tin, D, 3>), grid, dim3(kHqThreads), 0, s, X, V, eps, codes, d_out); break;
        case 4: hipLaunchKernelGGL((head_quant_kernel<Tin, D, 4>), grid, dim3(kHqThreads), 0, s, X, V, eps, codes, d_out); break;
        case 8: hipLaunchKernelGGL((head_quant_kernel<Tin, D, 8>), grid, dim3(kHqThreads), 0, s, X, V, eps, codes, d_out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_t(const Tin* X, int64_t V, int64_t D, int bits, float eps, uint8_t* codes, float* d_out,
                    hipStream_t s) {
    switch (D) {
        case 32: return launch_d<Tin, 32>(X, V, bits, eps, codes, d_out, s);
        case 64: return launch_d<Tin, 64>(X, V, bits, eps, codes, d_out, s);
        case 128: return launch_d<Tin, 128>(X, V, bits, eps, codes, d_out, s);
        case 256: return launch_d<Tin, 256>(X, V, bits, eps, codes, d_out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_head_quant(const void* X, int x_dtype, int64_t V, int64_t D, int bits, float eps, uint8_t* codes,
                             float* d_out, hipStream_t s) {
    if (V == 0) return hipSuccess;
    if (x_dtype == HBL_F32) return launch_t<float>((const float*)X, V, D, bits, eps, codes, d_out, s);
    return launch_t<uint16_t>((const uint16_t*)X, V, D, bits, eps, codes, d_out, s);
}

}  // namespace hbl
