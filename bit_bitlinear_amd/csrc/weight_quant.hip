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
//   wq_pack:    every wave issues its weight loads, then re-sums the
//               partials in one fixed order while they are in flight,
//               derives alpha = sum/(N*K) rounded to fp32, and each thread
//               turns two aligned groups of 16 weights into two 32-bit words.
//
// Ternary decision without a division.  With den = alpha + eps > 0 the code
// is round_half_even(w/den) clamped to [-1, 1], so it is 0 exactly when the
// correctly rounded quotient fl(|w|/den) is <= 1/2.  0.5 is an fp32 value
// whose upper neighbour is 0.5 + 2^-24, so fl(q) <= 1/2 iff q <= 0.5 + 2^-25,
// i.e. |w| <= den/2 * (1 + 2^-24).  When den/2 is a normal number the next
// fp32 value above den/2 exceeds that bound, so for fp32 w the test is just
// |w| <= den/2 (den/2 is exact).  Otherwise (den/2 subnormal, den infinite
// or NaN) the kernel divides as the definition does.  NaN weights give -1 on
// both paths (the clamp returns its non-NaN operand).
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int kWqThreads = 256;
constexpr int kMaxPartials = 512;
// Elements per wq_partial block are a multiple of this (keeps 16-byte vectors aligned).
constexpr int64_t kPartialQuantum = 4096;
constexpr int kRoundVecs = 8;     // 16-byte loads per thread issued together in wq_partial
constexpr int kPackGroups = 2;    // 16-weight groups per thread in wq_pack

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

HBL_DEVINL void unpack16(const uint4 q, float (&v)[4]) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
}
HBL_DEVINL void unpack16(const uint4 q, float (&v)[8]) {
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
    const int64_t n = min(count, begin + per_block) - begin;
    constexpr int64_t R = (int64_t)kRoundVecs * kWqThreads * V;  // elements per round
    double s = 0.0;
    for (int64_t r0 = 0; r0 < n; r0 += R) {
        // elements past this block's slice load as zeros, which add nothing
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + begin + r0, min(R, n - r0) * (int64_t)sizeof(T));
        uint4 q[kRoundVecs];
#pragma unroll
        for (int u = 0; u < kRoundVecs; u++) q[u] = buf_load16(rs, (uint32_t)((u * kWqThreads + threadIdx.x) * 16));
#pragma unroll
        for (int u = 0; u < kRoundVecs; u++) {
            float v[V];
            unpack16(q[u], v);
#pragma unroll
            for (int j = 0; j < V; j++) s += (double)fabsf(v[j]);
        }
    }
    s = block_sum_f64<kWqThreads>(s, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// 2-bit code of a ternary value: 0 -> 00, +1 -> 01, -1 -> 11.
HBL_DEVINL uint32_t tern_code_div(float w, float den) {
    // correctly rounded fp32 division, then round half to even, then clamp
    const float r = fminf(fmaxf(rintf(w / den), -1.f), 1.f);
    return r == 0.f ? 0u : (r > 0.f ? 1u : 3u);
}
HBL_DEVINL uint32_t tern_code_cmp(float w, float half_den) {
    return fabsf(w) <= half_den ? 0u : (w > 0.f ? 1u : 3u);
}

template <typename T>
__global__ __launch_bounds__(kWqThreads) void wq_pack(const T* __restrict__ W, int64_t n_groups, int64_t count,
                                                      float eps, const double* __restrict__ partial, int n_partial,
                                                      uint32_t* __restrict__ Wp, float* __restrict__ alpha_out) {
    constexpr int V = Vec16<T>::n;
    constexpr int kVecs = kPackGroups * 16 / V;  // 16-byte loads per thread
    constexpr int64_t kBlockGroups = (int64_t)kWqThreads * kPackGroups;
    const int64_t gb = (int64_t)blockIdx.x * kBlockGroups;  // first group of this block
    const int64_t g0 = gb + (int64_t)threadIdx.x * kPackGroups;
    // groups past the end load as zeros and their words are not stored
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + gb * 16, min(kBlockGroups, n_groups - gb) * 16 * (int64_t)sizeof(T));
    uint4 q[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; u++) q[u] = buf_load16(rs, (uint32_t)((threadIdx.x * kVecs + u) * 16));

    // Every wave sums all partials in the same fixed order (lane l takes
    // l, l+64, ... in turn, then a butterfly), so all waves of all blocks
    // derive the same alpha without a block barrier.
    const int lane = threadIdx.x & (kWave - 1);
    double s = 0.0;
    for (int i = lane; i < n_partial; i += kWave) s += partial[i];
    s = wave_sum_f64(s);
    const float alpha = (float)(s / (double)count);
    if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_out = alpha;
    const float den = alpha + eps;
    const float half_den = den * 0.5f;
    const bool fast = half_den >= 1.17549435e-38f && den <= 3.40282347e38f;  // den/2 normal, den finite

    uint32_t word[kPackGroups];
#pragma unroll
    for (int gi = 0; gi < kPackGroups; gi++) {
        float v[16];
#pragma unroll
        for (int c = 0; c < 16 / V; c++) {
            float t[V];
            unpack16(q[gi * (16 / V) + c], t);
#pragma unroll
            for (int j = 0; j < V; j++) v[c * V + j] = t[j];
        }
        uint32_t w = 0;
        // element e of the group -> byte e%4, bit pair e/4
        if (fast) {
#pragma unroll
            for (int e = 0; e < 16; e++) w |= tern_code_cmp(v[e], half_den) << (8 * (e & 3) + 2 * (e >> 2));
        } else if (den != 0.f) {
#pragma unroll
            for (int e = 0; e < 16; e++) w |= tern_code_div(v[e], den) << (8 * (e & 3) + 2 * (e >> 2));
        }
        word[gi] = w;
    }
    if (g0 + kPackGroups <= n_groups) {
        *reinterpret_cast<uint2*>(Wp + g0) = make_uint2(word[0], word[1]);
    } else {
#pragma unroll
        for (int gi = 0; gi < kPackGroups; gi++)
            if (g0 + gi < n_groups) Wp[g0 + gi] = word[gi];
    }
}
static_assert(kPackGroups == 2, "the vector store above writes two words");

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
    const int64_t blocks = (n_groups + (int64_t)kWqThreads * kPackGroups - 1) / ((int64_t)kWqThreads * kPackGroups);
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
