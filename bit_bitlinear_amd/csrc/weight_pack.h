// weight_pack.h -- the packing half of the per-tensor absmean ternarisation
// (gfx950), as a block routine shared by the standalone packing kernel and
// the fused activation + packing kernel.  Internal header.
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块" (one
// absmean scale per tensor, weights in {-1, 0, 1}); the zero band is
// inclusive as on the CSDN blog "[论文品鉴] 1-bit LLM", section "量化函数".
//
// Ternary decision without a division.  With den = alpha + eps > 0 the code
// is round_half_even(w/den) clamped to [-1, 1], so it is 0 exactly when the
// correctly rounded quotient fl(|w|/den) is <= 1/2.  0.5 is an fp32 value
// whose upper neighbour is 0.5 + 2^-24, so fl(q) <= 1/2 iff q <= 0.5 + 2^-25,
// i.e. |w| <= den/2 * (1 + 2^-24).  When den/2 is a normal number the next
// fp32 value above den/2 exceeds that bound, so for fp32 w the test is just
// |w| <= den/2 (den/2 is exact).  Otherwise (den/2 subnormal, den infinite
// or NaN) the routine divides as the definition does.  NaN weights give -1 on
// both paths (the clamp returns its non-NaN operand).
#pragma once
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int kPackGroups = 2;  // 16-weight groups per thread

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

// Partial |W| sums.  Block blk sums |W| over elements [blk*per_block,
// (blk+1)*per_block) in fp64 in one fixed order, the order of a block of
// kPartialVThreads threads: in every round of kPartialRoundVecs*256 16-byte
// vectors, virtual thread t adds the elements of vectors u*256 + t (u
// ascending, elements in order), then each 64-thread virtual wave is summed
// by wave_sum_f64 and the wave sums are added in wave order, as
// block_sum_f64 does.  A block of NT real threads (NT a multiple of 64
// dividing 256) plays 256/NT virtual threads per thread (virtual thread
// h*NT + tid), so the result does not depend on NT: the standalone launch
// (256 threads) and the 64-thread blocks that share a grid with the
// activation rows write the same partial sums bit for bit.
// red: kPartialVThreads/64 doubles of LDS.
constexpr int kPartialVThreads = 256;
constexpr int kPartialRoundVecs = 8;  // 16-byte loads per virtual thread and round

template <typename T, int NT>
HBL_DEVINL void wq_partial_block(const T* __restrict__ W, int64_t count, int64_t per_block,
                                 double* __restrict__ partial, int64_t blk, double* red) {
    static_assert(NT % kWave == 0 && kPartialVThreads % NT == 0, "thread count");
    constexpr int V = Vec16<T>::n;
    constexpr int VT = kPartialVThreads / NT;   // virtual threads per thread
    constexpr int HB = VT >= 2 ? 2 : 1;         // virtual threads whose loads are issued together
    const int64_t begin = blk * per_block;
    const int64_t n = min(count, begin + per_block) - begin;
    constexpr int64_t R = (int64_t)kPartialRoundVecs * kPartialVThreads * V;  // elements per round
    double s[VT];
#pragma unroll
    for (int h = 0; h < VT; h++) s[h] = 0.0;
    for (int64_t r0 = 0; r0 < n; r0 += R) {
        // elements past this block's slice load as zeros, which add nothing
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + begin + r0, min(R, n - r0) * (int64_t)sizeof(T));
#pragma unroll
        for (int h0 = 0; h0 < VT; h0 += HB) {
            uint4 q[HB][kPartialRoundVecs];
#pragma unroll
            for (int h = 0; h < HB; h++)
#pragma unroll
                for (int u = 0; u < kPartialRoundVecs; u++)
                    q[h][u] = buf_load16(
                        rs, (uint32_t)((u * kPartialVThreads + (h0 + h) * NT + (int)threadIdx.x) * 16));
#pragma unroll
            for (int h = 0; h < HB; h++)
#pragma unroll
                for (int u = 0; u < kPartialRoundVecs; u++) {
                    float v[V];
                    unpack16(q[h][u], v);
#pragma unroll
                    for (int j = 0; j < V; j++) s[h0 + h] += (double)fabsf(v[j]);
                }
        }
    }
#pragma unroll
    for (int h = 0; h < VT; h++) {
        const double w = wave_sum_f64(s[h]);
        if ((threadIdx.x & (kWave - 1)) == 0) red[h * (NT / kWave) + threadIdx.x / kWave] = w;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double r = 0.0;
#pragma unroll
        for (int i = 0; i < kPartialVThreads / kWave; i++) r += red[i];
        partial[blk] = r;
    }
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

// One packing block of NT threads: groups [blk * 2NT, (blk+1) * 2NT) of the
// N*K/16 aligned 16-weight groups.  Every wave re-sums the partial |W| sums
// in one fixed order (lane l takes l, l+64, ..., then a butterfly), so all
// waves of all blocks derive the same alpha with no block barrier; block 0
// also stores alpha.  The weight loads are issued before that re-sum.
template <typename T, int NT>
HBL_DEVINL void wq_pack_block(const T* __restrict__ W, int64_t n_groups, int64_t count, float eps,
                              const double* __restrict__ partial, int n_partial, uint32_t* __restrict__ Wp,
                              float* __restrict__ alpha_out, int64_t blk) {
    constexpr int V = Vec16<T>::n;
    constexpr int kVecs = kPackGroups * 16 / V;  // 16-byte loads per thread
    constexpr int64_t kBlockGroups = (int64_t)NT * kPackGroups;
    const int64_t gb = blk * kBlockGroups;  // first group of this block
    const int64_t g0 = gb + (int64_t)threadIdx.x * kPackGroups;
    // groups past the end load as zeros and their words are not stored
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(W + gb * 16, min(kBlockGroups, n_groups - gb) * 16 * (int64_t)sizeof(T));
    uint4 q[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; u++) q[u] = buf_load16(rs, (uint32_t)((threadIdx.x * kVecs + u) * 16));

    const int lane = threadIdx.x & (kWave - 1);
    double s = 0.0;
    for (int i = lane; i < n_partial; i += kWave) s += partial[i];
    s = wave_sum_f64(s);
    const float alpha = (float)(s / (double)count);
    if (blk == 0 && threadIdx.x == 0) *alpha_out = alpha;
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
}  // namespace hbl
