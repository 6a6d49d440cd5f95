// weight_quant.hip -- per-tensor absmean ternarisation of latent weights and
// packing into the library's 2-bit format (gfx950).
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块": the
// weights are ternarised to {-1, 0, 1} with one absmean scale per tensor.
// The threshold form on the CSDN blog "[论文品鉴] 1-bit LLM", section "量化函数",
// fixes the zero band as inclusive, which round-half-to-even reproduces.
//
// Two launches, both HBM-bound streams over W:
//   wq_partial: block b sums |W| over a fixed contiguous slice in fp64
//               (fixed order, so alpha is deterministic run to run);
//   wq_pack:    every block re-sums the partials in the same fixed order,
//               derives alpha = sum/(N*K) rounded to fp32, and each thread
//               ternarises one aligned group of 16 weights into one 32-bit word.
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int kWqThreads = 256;
constexpr int kMaxPartials = 1024;
// Elements per wq_partial block are a multiple of this (keeps 16-byte vectors aligned).
constexpr int64_t kPartialQuantum = 4096;

template <typename T>
struct Vec16;  // 16-byte vector of weights
template <>
struct Vec16<float> {
    static constexpr int n = 4;
};
template <>
struct Vec16<uint16_t> {
    static constexpr int n = 8;
};

HBL_DEVINL void load16(const float* p, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
HBL_DEVINL void load16(const uint16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

template <typename T>
__global__ __launch_bounds__(kWqThreads) void wq_partial(const T* __restrict__ W, int64_t count, int64_t per_block,
                                                         double* __restrict__ partial) {
    __shared__ double red[kWqThreads / kWave];
    constexpr int V = Vec16<T>::n;
    const int64_t begin = (int64_t)blockIdx.x * per_block;
    const int64_t end = min(count, begin + per_block);
    double s = 0.0;
    for (int64_t i = begin + (int64_t)threadIdx.x * V; i < end; i += (int64_t)kWqThreads * V) {
        float v[V];
        load16(W + i, v);
#pragma unroll
        for (int j = 0; j < V; j++) s += (double)fabsf(v[j]);
    }
    s = block_sum_f64<kWqThreads>(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// 2-bit code of a ternary value: 0 -> 00, +1 -> 01, -1 -> 11.
HBL_DEVINL uint32_t tern_code(float w, float den) {
    // den > 0 here; correctly rounded fp32 division, then round half to even.
    const float r = fminf(fmaxf(rintf(w / den), -1.f), 1.f);
    return r == 0.f ? 0u : (r > 0.f ? 1u : 3u);
}

template <typename T>
__global__ __launch_bounds__(kWqThreads) void wq_pack(const T* __restrict__ W, int64_t n_groups, int64_t count,
                                                      float eps, const double* __restrict__ partial, int n_partial,
                                                      uint32_t* __restrict__ Wp, float* __restrict__ alpha_out) {
    __shared__ double red[kWqThreads / kWave];
    double s = 0.0;
    for (int i = threadIdx.x; i < n_partial; i += kWqThreads) s += partial[i];
    s = block_sum_f64<kWqThreads>(s, red);
    const float alpha = (float)(s / (double)count);
    if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_out = alpha;
    const float den = alpha + eps;

    constexpr int V = Vec16<T>::n;
    for (int64_t g = (int64_t)blockIdx.x * kWqThreads + threadIdx.x; g < n_groups;
         g += (int64_t)gridDim.x * kWqThreads) {
        float v[16];
#pragma unroll
        for (int c = 0; c < 16 / V; c++) {
            float t[V];
            load16(W + g * 16 + c * V, t);
#pragma unroll
            for (int j = 0; j < V; j++) v[c * V + j] = t[j];
        }
        uint32_t word = 0;
        if (den != 0.f) {
            // element e of the group -> byte e%4, bit pair e/4
#pragma unroll
            for (int e = 0; e < 16; e++) word |= tern_code(v[e], den) << (8 * (e & 3) + 2 * (e >> 2));
        }
        Wp[g] = word;
    }
}

}  // namespace

int weight_partial_count(int64_t count) {
    int64_t per = (count + kMaxPartials - 1) / kMaxPartials;
    per = (per + kPartialQuantum - 1) / kPartialQuantum * kPartialQuantum;
    return (int)((count + per - 1) / per);
}

hipError_t launch_weight_quant(const void* W, int w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                               float* alpha, double* partial, int n_partial, hipStream_t s) {
    const int64_t count = N * K;
    int64_t per = (count + kMaxPartials - 1) / kMaxPartials;
    per = (per + kPartialQuantum - 1) / kPartialQuantum * kPartialQuantum;
    const int64_t n_groups = count / 16;
    int64_t blocks = (n_groups + kWqThreads - 1) / kWqThreads;
    if (blocks > 4096) blocks = 4096;
    if (w_dtype == HBL_F32) {
        hipLaunchKernelGGL(wq_partial<float>, dim3(n_partial), dim3(kWqThreads), 0, s, (const float*)W, count, per,
                           partial);
        hipLaunchKernelGGL(wq_pack<float>, dim3((unsigned)blocks), dim3(kWqThreads), 0, s, (const float*)W, n_groups,
                           count, eps, (const double*)partial, n_partial, (uint32_t*)W_packed, alpha);
    } else {
        hipLaunchKernelGGL(wq_partial<uint16_t>, dim3(n_partial), dim3(kWqThreads), 0, s, (const uint16_t*)W, count,
                           per, partial);
        hipLaunchKernelGGL(wq_pack<uint16_t>, dim3((unsigned)blocks), dim3(kWqThreads), 0, s, (const uint16_t*)W,
                           n_groups, count, eps, (const double*)partial, n_partial, (uint32_t*)W_packed, alpha);
    }
    return hipGetLastError();
}

}  // namespace hbl
