// act_pack.hip -- one launch that runs the per-token activation quantisation
// (norm, online Hadamard, per-token scale, codes) side by side with one half
// of the per-tensor absmean ternarisation of the weights (gfx950).
//
// The codes need only X; the partial |W| sums need only W, and the packed
// weights only W and those sums.  On one stream each would otherwise be a
// launch of its own, and at the sizes of one layer all of them are bound by
// launch and memory latency rather than by throughput, so sharing a grid
// overlaps them.  M blocks run the row routine of act_row.h (the same code
// and thread count as the standalone activation kernel, so codes and scales
// are bit-identical); the other blocks run, with the same thread count,
// either the partial-sum block routine of weight_pack.h (which reproduces
// the standalone launch's summation order, so alpha is bit-identical) or its
// packing block routine (each packed word depends only on its 16 weights and
// alpha).  hbl_forward_latent uses the first form: rows and partial sums
// here, then the packing launch, which measured faster than the partial sums
// first and rows with packing after (1.3B Wo step 38.4 -> 36.8 us of kernel
// time).  The two kinds of block are interleaved over the grid.
// Rows up to 2048 elements only (longer rows keep the launches separate).
// The codes go out in one of the layouts of hbl_device.h (row-major, decode
// tiles or FP6).
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块".
#include "act_row.h"
#include "weight_pack.h"
#include "lds_attr.h"

namespace hbl {
namespace {

template <int LK, int NT, typename Tin, int BITS, bool HAD, typename TW, int LAYOUT>
__global__ __launch_bounds__(NT) void act_pack_kernel(const Tin* __restrict__ X, int64_t M,
                                                      const float* __restrict__ gain, int norm, float norm_eps,
                                                      float quant_eps, int a4_mode, uint8_t* __restrict__ codes,
                                                      float* __restrict__ xscale, const TW* __restrict__ W,
                                                      int64_t n_groups, int64_t count, float w_eps,
                                                      const double* __restrict__ partial, int n_partial,
                                                      int64_t per_block, double* __restrict__ partial_out,
                                                      uint32_t* __restrict__ Wp, float* __restrict__ alpha) {
    using S = ActShape<LK, NT, Tin>;
    extern __shared__ __attribute__((aligned(16))) float lds[];  // float4 accesses
    __shared__ ActPartF<LK, NT, Tin> partf;
    __shared__ ActPartD<LK, NT, Tin> partd;
    // The P weight blocks are spread evenly among the M + P blocks (blocks
    // are dispatched in index order, so a contiguous range of either kind
    // would run mostly alone): block b is a weight block iff floor((b+1)P/T) > floor(bP/T);
    // floor(bP/T) blocks before it pack, so b is row b - floor(bP/T) or
    // packing block floor(bP/T).
    const int64_t b = blockIdx.x, T = (int64_t)gridDim.x, P = T - M;
    const int64_t p_lo = b * P / T, p_hi = (b + 1) * P / T;
    if (p_hi == p_lo) {
        const int64_t row = b - p_lo;
        ActRegs<LK, NT, Tin> v;
        act_row_load<LK, NT, Tin>(X + row * S::K, v);
        const Fp6RowPlace f6 = LAYOUT == kCodesFp6 ? fp6_row_place(row, M, S::K) : Fp6RowPlace{0, 96, 0};
        uint8_t* const crow = codes + (LAYOUT == kCodesDecTiled ? dec_tile_row_base<BITS>(row, S::K)
                                       : LAYOUT == kCodesFp6    ? f6.base
                                                                : row * (S::K * BITS / 8));
        act_row_quantise<LK, NT, Tin, BITS, HAD, LAYOUT>(v, gain, norm, norm_eps, quant_eps, a4_mode, lds, partf,
                                                        partd, crow, xscale + row, nullptr, nullptr, f6.stride,
                                                        f6.swz);
    } else if (partial_out) {
        __shared__ double red[kPartialVThreads / kWave];
        wq_partial_block<TW, NT>(W, count, per_block, partial_out, p_lo, red);
    } else {
        wq_pack_block<TW, NT>(W, n_groups, count, w_eps, partial, n_partial, Wp, alpha, p_lo);
    }
}

template <int LK, typename Tin, int BITS, bool HAD, typename TW, int LAYOUT>
hipError_t launch_ap(const Tin* X, int64_t M, const float* gain, const hbl_config& cfg, void* codes, float* xscale,
                     const TW* W, int64_t NK, float w_eps, const double* partial, double* partial_out, int n_partial, uint8_t* Wp,
                     float* alpha, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    // the Hadamard's fp32 row; the FP6 layout stages one dword per four codes there too
    const size_t row_bytes = HAD ? (size_t)ActShape<LK, NT, Tin>::lds_floats * sizeof(float) : 0;
    const size_t lds_bytes = LAYOUT == kCodesFp6 && row_bytes < (size_t)(1 << LK) ? (size_t)(1 << LK) : row_bytes;
    auto kern = act_pack_kernel<LK, NT, Tin, BITS, HAD, TW, LAYOUT>;
    static std::atomic<uint32_t> lds_set{0};  // devices with the LDS limit raised for this kernel
    if (hipError_t e = set_dynamic_lds(kern, lds_bytes, lds_set); e != hipSuccess) return e;
    const int64_t n_groups = NK / 16;
    const int64_t pack_blocks = (n_groups + 2 * NT - 1) / (2 * NT);
    const int64_t grid = M + (partial_out ? (int64_t)n_partial : pack_blocks);
    const int64_t per_block = weight_partial_slice(NK);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds_bytes, s, X, M, gain, cfg.norm, cfg.norm_eps,
                       cfg.quant_eps, cfg.a4_mode, (uint8_t*)codes, xscale, W, n_groups, NK, w_eps, partial,
                       n_partial, per_block, partial_out, (uint32_t*)Wp, alpha);
    return hipGetLastError();
}

template <typename Tin, int BITS, bool HAD, typename TW, int LAYOUT>
hipError_t dispatch_k(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                      float* xscale, const TW* W, int64_t NK, float w_eps, const double* partial, double* partial_out, int n_partial,
                      uint8_t* Wp, float* alpha, hipStream_t s) {
#define HBL_AP(LK) \
    launch_ap<LK, Tin, BITS, HAD, TW, LAYOUT>(X, M, gain, cfg, codes, xscale, W, NK, w_eps, partial, partial_out, n_partial, Wp, alpha, s)
    switch (K) {
        case 256:
            if constexpr (LAYOUT == kCodesFp6) return hipErrorInvalidValue;  // two values per vector
            else return HBL_AP(8);
        case 512: return HBL_AP(9);
        case 1024: return HBL_AP(10);
        case 2048: return HBL_AP(11);
        default: return hipErrorInvalidValue;
    }
#undef HBL_AP
}

template <typename Tin, int BITS, bool HAD, typename TW>
hipError_t dispatch_layout(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg,
                           void* codes, float* xscale, const TW* W, int64_t NK, float w_eps, const double* partial, double* partial_out,
                           int n_partial, uint8_t* Wp, float* alpha, hipStream_t s, int layout) {
#define HBL_APL(L) dispatch_k<Tin, BITS, HAD, TW, L>(X, M, K, gain, cfg, codes, xscale, W, NK, w_eps, partial, partial_out, n_partial, Wp, alpha, s)
    switch (layout) {
        case kCodesRowMajor: return HBL_APL(kCodesRowMajor);
        case kCodesDecTiled: return HBL_APL(kCodesDecTiled);
        case kCodesFp6:
            if constexpr (BITS == 4) return HBL_APL(kCodesFp6);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
#undef HBL_APL
}

template <typename Tin, typename TW>
hipError_t dispatch_mode(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                         float* xscale, const TW* W, int64_t NK, float w_eps, const double* partial, double* partial_out, int n_partial,
                         uint8_t* Wp, float* alpha, hipStream_t s, int layout) {
    if (cfg.act_bits == 8)
        return cfg.hadamard ? dispatch_layout<Tin, 8, true, TW>(X, M, K, gain, cfg, codes, xscale, W, NK, w_eps,
                                                              partial, partial_out, n_partial, Wp, alpha, s, layout)
                            : dispatch_layout<Tin, 8, false, TW>(X, M, K, gain, cfg, codes, xscale, W, NK, w_eps,
                                                               partial, partial_out, n_partial, Wp, alpha, s, layout);
    return cfg.hadamard ? dispatch_layout<Tin, 4, true, TW>(X, M, K, gain, cfg, codes, xscale, W, NK, w_eps, partial, partial_out,
                                                          n_partial, Wp, alpha, s, layout)
                        : dispatch_layout<Tin, 4, false, TW>(X, M, K, gain, cfg, codes, xscale, W, NK, w_eps, partial, partial_out,
                                                           n_partial, Wp, alpha, s, layout);
}

template <typename Tin>
hipError_t dispatch_w(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                      float* xscale, const void* W, int w_dtype, int64_t NK, float w_eps, const double* partial, double* partial_out,
                      int n_partial, uint8_t* Wp, float* alpha, hipStream_t s, int layout) {
    if (w_dtype == HBL_F32)
        return dispatch_mode<Tin, float>(X, M, K, gain, cfg, codes, xscale, (const float*)W, NK, w_eps, partial, partial_out,
                                         n_partial, Wp, alpha, s, layout);
    return dispatch_mode<Tin, uint16_t>(X, M, K, gain, cfg, codes, xscale, (const uint16_t*)W, NK, w_eps, partial, partial_out,
                                        n_partial, Wp, alpha, s, layout);
}

}  // namespace

hipError_t launch_act_and_pack(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                               const hbl_config& cfg, void* codes, float* xscale, const void* W, int w_dtype,
                               int64_t NK, float w_eps, const double* partial, double* partial_out, int n_partial, uint8_t* W_packed,
                               float* alpha, hipStream_t s, int layout) {
    if (x_dtype == HBL_F32)
        return dispatch_w<float>((const float*)X, M, K, gain, cfg, codes, xscale, W, w_dtype, NK, w_eps, partial, partial_out,
                                 n_partial, W_packed, alpha, s, layout);
    return dispatch_w<uint16_t>((const uint16_t*)X, M, K, gain, cfg, codes, xscale, W, w_dtype, NK, w_eps, partial, partial_out,
                                n_partial, W_packed, alpha, s, layout);
}

}  // namespace hbl
