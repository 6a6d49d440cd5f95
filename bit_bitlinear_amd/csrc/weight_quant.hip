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
//               (fixed order, so alpha is deterministic run to run); every
//               thread issues all its 16-byte loads of one round before it
//               adds anything;
//   wq_pack:    the block routine of weight_pack.h: every wave issues its
//               weight loads, then re-sums the partials in one fixed order
//               while they are in flight, derives alpha = sum/(N*K) rounded
//               to fp32, and each thread turns two aligned groups of 16
//               weights into two 32-bit words.
//
// The ternary decision is division-free (see weight_pack.h).
#include "weight_pack.h"

namespace hbl {
namespace {

constexpr int kWqThreads = 256;
constexpr int kMaxPartials = 512;
// Elements per wq_partial block are a multiple of this (keeps 16-byte vectors aligned).
constexpr int64_t kPartialQuantum = 4096;

template <typename T>
__global__ __launch_bounds__(kWqThreads) void wq_partial(const T* __restrict__ W, int64_t count, int64_t per_block,
                                                         double* __restrict__ partial) {
    __shared__ double red[kPartialVThreads / kWave];
    wq_partial_block<T, kWqThreads>(W, count, per_block, partial, blockIdx.x, red);
}

template <typename T>
__global__ __launch_bounds__(kWqThreads) void wq_pack(const T* __restrict__ W, int64_t n_groups, int64_t count,
                                                      float eps, const double* __restrict__ partial, int n_partial,
                                                      uint32_t* __restrict__ Wp, float* __restrict__ alpha_out) {
    wq_pack_block<T, kWqThreads>(W, n_groups, count, eps, partial, n_partial, Wp, alpha_out, blockIdx.x);
}

}  // namespace

namespace {
int64_t partial_slice(int64_t count) {
    int64_t per = (count + kMaxPartials - 1) / kMaxPartials;
    return (per + kPartialQuantum - 1) / kPartialQuantum * kPartialQuantum;
}
}  // namespace

int64_t weight_partial_slice(int64_t count) { return partial_slice(count); }

int weight_partial_count(int64_t count) {
    const int64_t per = partial_slice(count);
    return (int)((count + per - 1) / per);
}

hipError_t launch_weight_partial(const void* W, int w_dtype, int64_t count, double* partial, int n_partial,
                                 hipStream_t s) {
    const int64_t per = partial_slice(count);
    if (w_dtype == HBL_F32)
        hipLaunchKernelGGL(wq_partial<float>, dim3(n_partial), dim3(kWqThreads), 0, s, (const float*)W, count, per,
                           partial);
    else
        hipLaunchKernelGGL(wq_partial<uint16_t>, dim3(n_partial), dim3(kWqThreads), 0, s, (const uint16_t*)W, count,
                           per, partial);
    return hipGetLastError();
}

hipError_t launch_weight_pack(const void* W, int w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                              float* alpha, const double* partial, int n_partial, hipStream_t s) {
    const int64_t count = N * K;
    const int64_t n_groups = count / 16;
    const int64_t blocks = (n_groups + (int64_t)kWqThreads * kPackGroups - 1) / ((int64_t)kWqThreads * kPackGroups);
    if (w_dtype == HBL_F32)
        hipLaunchKernelGGL(wq_pack<float>, dim3((unsigned)blocks), dim3(kWqThreads), 0, s, (const float*)W, n_groups,
                           count, eps, partial, n_partial, (uint32_t*)W_packed, alpha);
    else
        hipLaunchKernelGGL(wq_pack<uint16_t>, dim3((unsigned)blocks), dim3(kWqThreads), 0, s, (const uint16_t*)W,
                           n_groups, count, eps, partial, n_partial, (uint32_t*)W_packed, alpha);
    return hipGetLastError();
}

hipError_t launch_weight_quant(const void* W, int w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                               float* alpha, double* partial, int n_partial, hipStream_t s) {
    hipError_t e = launch_weight_partial(W, w_dtype, N * K, partial, n_partial, s);
    if (e != hipSuccess) return e;
    return launch_weight_pack(W, w_dtype, N, K, eps, W_packed, alpha, partial, n_partial, s);
}

}  // namespace hbl
