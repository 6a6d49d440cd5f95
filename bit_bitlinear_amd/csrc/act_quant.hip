// act_quant.hip -- fused per-token RMSNorm/LayerNorm + online fast Walsh-Hadamard
// transform + INT8/INT4 quantisation and packing (gfx950): one workgroup per
// token row running the row routine of act_row.h (which cites the passages
// it follows and describes the register / LDS layout).  The codes go out in
// one of the layouts of hbl_device.h: the ABI's row-major one, the decode
// tile layout (for the decode GEMM) or FP6 (for the FP6 x FP4 GEMM).
#include "act_row.h"
#include "lds_attr.h"

namespace hbl {
namespace {

// PLAIN: the default configuration (RMSNorm, the absmean INT4 statistic, no
// gain, no debug outputs) with every other path compiled out of the row
// routine: 8-13% faster than the general kernel, which tests the norm, the
// statistic and the pointers at run time (3B-like layer shapes, K = 2048 to
// 16384).
template <int LK, int NT, typename Tin, int BITS, bool HAD, int LAYOUT, bool PLAIN>
__global__ __launch_bounds__(NT) void act_quant_kernel(const Tin* __restrict__ X, int64_t M,
                                                       const float* __restrict__ gain, int norm, float norm_eps,
                                                       float quant_eps, int a4_mode, uint8_t* __restrict__ codes,
                                                       float* __restrict__ xscale, float* __restrict__ z_debug,
                                                       float* __restrict__ s_debug) {
    using S = ActShape<LK, NT, Tin>;
    extern __shared__ __attribute__((aligned(16))) float lds[];  // float4 accesses
    __shared__ ActPartF<LK, NT, Tin> partf;
    __shared__ ActPartD<LK, NT, Tin> partd;
    // FP6 codes: rows are dealt to the XCDs in contiguous ranges (block b runs
    // on XCD b % 8), so that the 96-byte pieces of neighbouring rows, which
    // share cache lines in the FP6 layout, meet in one L2
    const int64_t b = blockIdx.x;
    const int64_t row = LAYOUT == kCodesFp6 && M % 8 == 0 ? (b % 8) * (M / 8) + b / 8 : b;
    ActRegs<LK, NT, Tin> v;
    act_row_load<LK, NT, Tin>(X + row * S::K, v);
    const Fp6RowPlace f6 = LAYOUT == kCodesFp6 ? fp6_row_place(row, M, S::K) : Fp6RowPlace{0, 96, 0};
    uint8_t* const crow = codes + (LAYOUT == kCodesDecTiled ? dec_tile_row_base<BITS>(row, S::K)
                                   : LAYOUT == kCodesFp6    ? f6.base
                                                            : row * (S::K * BITS / 8));
    if constexpr (PLAIN)
        act_row_quantise<LK, NT, Tin, BITS, HAD, LAYOUT>(v, nullptr, (int)HBL_NORM_RMS, norm_eps, quant_eps,
                                                        (int)HBL_A4_ABSMEAN_SQRT7, lds, partf, partd, crow,
                                                        xscale + row, nullptr, nullptr, f6.stride, f6.swz);
    else
        act_row_quantise<LK, NT, Tin, BITS, HAD, LAYOUT>(v, gain, norm, norm_eps, quant_eps, a4_mode, lds, partf,
                                                        partd, crow, xscale + row,
                                                        z_debug ? z_debug + row * S::K : nullptr,
                                                        s_debug ? s_debug + row : nullptr, f6.stride, f6.swz);
}

template <int LK, typename Tin, int BITS, bool HAD, int LAYOUT, bool PLAIN>
hipError_t launch_one_as(const Tin* X, int64_t M, const float* gain, const hbl_config& cfg, void* codes,
                         float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    // the Hadamard's fp32 row; the FP6 layout stages one dword per four codes there too
    const size_t row_bytes = HAD ? (size_t)ActShape<LK, NT, Tin>::lds_floats * sizeof(float) : 0;
    const size_t lds_bytes = LAYOUT == kCodesFp6 && row_bytes < (size_t)(1 << LK) ? (size_t)(1 << LK) : row_bytes;
    auto kern = act_quant_kernel<LK, NT, Tin, BITS, HAD, LAYOUT, PLAIN>;
    static std::atomic<uint32_t> lds_set{0};  // devices with the LDS limit raised for this kernel
    if (hipError_t e = set_dynamic_lds(kern, lds_bytes, lds_set); e != hipSuccess) return e;
    // one workgroup per row; gridDim.x is limited to 2^31-1
    hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(NT), lds_bytes, s, X, M, gain, cfg.norm, cfg.norm_eps,
                       cfg.quant_eps, cfg.a4_mode, (uint8_t*)codes, xscale, z_debug, s_debug);
    return hipGetLastError();
}

template <int LK, typename Tin, int BITS, bool HAD, int LAYOUT>
hipError_t launch_one(const Tin* X, int64_t M, const float* gain, const hbl_config& cfg, void* codes, float* xscale,
                      float* z_debug, float* s_debug, hipStream_t s) {
    if (!gain && !z_debug && !s_debug && cfg.norm == HBL_NORM_RMS && (BITS == 8 || cfg.a4_mode == HBL_A4_ABSMEAN_SQRT7))
        return launch_one_as<LK, Tin, BITS, HAD, LAYOUT, true>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
    return launch_one_as<LK, Tin, BITS, HAD, LAYOUT, false>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

template <typename Tin, int BITS, bool HAD, int LAYOUT>
hipError_t dispatch_k(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                      float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
#define HBL_AQ(LK) launch_one<LK, Tin, BITS, HAD, LAYOUT>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s)
    switch (K) {
        case 256:
            if constexpr (LAYOUT == kCodesFp6) return hipErrorInvalidValue;  // two values per vector
            else return HBL_AQ(8);
        case 512: return HBL_AQ(9);
        case 1024: return HBL_AQ(10);
        case 2048: return HBL_AQ(11);
        case 4096: return HBL_AQ(12);
        case 8192: return HBL_AQ(13);
        case 16384: return HBL_AQ(14);
        case 32768: return HBL_AQ(15);
        default: return hipErrorInvalidValue;
    }
#undef HBL_AQ
}

template <typename Tin, int LAYOUT>
hipError_t dispatch_mode(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                         float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    if (cfg.act_bits == 8) {
        if constexpr (LAYOUT == kCodesFp6) return hipErrorInvalidValue;  // FP6 holds INT4 codes only
        else
            return cfg.hadamard
                       ? dispatch_k<Tin, 8, true, LAYOUT>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                       : dispatch_k<Tin, 8, false, LAYOUT>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    }
    return cfg.hadamard ? dispatch_k<Tin, 4, true, LAYOUT>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                        : dispatch_k<Tin, 4, false, LAYOUT>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

template <int LAYOUT>
hipError_t dispatch_x(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain, const hbl_config& cfg,
                      void* codes, float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    if (x_dtype == HBL_F32)
        return dispatch_mode<float, LAYOUT>((const float*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    return dispatch_mode<uint16_t, LAYOUT>((const uint16_t*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

}  // namespace

hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                            const hbl_config& cfg, void* codes, float* xscale, float* z_debug, float* s_debug,
                            hipStream_t s, int layout) {
    if (M == 0) return hipSuccess;
    switch (layout) {
        case kCodesRowMajor:
            return dispatch_x<kCodesRowMajor>(X, x_dtype, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case kCodesDecTiled:
            return dispatch_x<kCodesDecTiled>(X, x_dtype, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case kCodesFp6:
            return dispatch_x<kCodesFp6>(X, x_dtype, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hbl
