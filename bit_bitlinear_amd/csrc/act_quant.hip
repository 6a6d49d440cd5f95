// act_quant.hip -- fused per-token RMSNorm/LayerNorm + online fast Walsh-Hadamard
// transform + INT8/INT4 quantisation and packing (gfx950): one workgroup per
// token row running the row routine of act_row.h (which cites the passages
// it follows and describes the register / LDS layout).  With TILED the codes
// are written in the decode tile layout of hbl_device.h (for the decode GEMM).
#include "act_row.h"

namespace hbl {
namespace {

template <int LK, int NT, typename Tin, int BITS, bool HAD, bool TILED>
__global__ __launch_bounds__(NT) void act_quant_kernel(const Tin* __restrict__ X, const float* __restrict__ gain,
                                                       int norm, float norm_eps, float quant_eps, int a4_mode,
                                                       uint8_t* __restrict__ codes, float* __restrict__ xscale,
                                                       float* __restrict__ z_debug, float* __restrict__ s_debug) {
    using S = ActShape<LK, NT, Tin>;
    extern __shared__ __attribute__((aligned(16))) float lds[];  // float4 accesses
    __shared__ ActPartF<LK, NT, Tin> partf;
    __shared__ ActPartD<LK, NT, Tin> partd;
    const int64_t row = blockIdx.x;
    ActRegs<LK, NT, Tin> v;
    act_row_load<LK, NT, Tin>(X + row * S::K, v);
    uint8_t* const crow = codes + (TILED ? dec_tile_row_base<BITS>(row, S::K) : row * (S::K * BITS / 8));
    act_row_quantise<LK, NT, Tin, BITS, HAD, TILED>(v, gain, norm, norm_eps, quant_eps, a4_mode, lds, partf, partd,
                                                    crow, xscale + row,
                                             z_debug ? z_debug + row * S::K : nullptr, s_debug ? s_debug + row : nullptr);
}

template <int LK, typename Tin, int BITS, bool HAD, bool TILED>
hipError_t launch_one(const Tin* X, int64_t M, const float* gain, const hbl_config& cfg, void* codes, float* xscale,
                      float* z_debug, float* s_debug, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    const size_t lds_bytes = HAD ? (size_t)ActShape<LK, NT, Tin>::lds_floats * sizeof(float) : 0;
    auto kern = act_quant_kernel<LK, NT, Tin, BITS, HAD, TILED>;
    static bool attr_set = false;  // one attribute call per instantiation
    if (!attr_set && lds_bytes > 0) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // one workgroup per row; gridDim.x is limited to 2^31-1
    hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(NT), lds_bytes, s, X, gain, cfg.norm, cfg.norm_eps,
                       cfg.quant_eps, cfg.a4_mode, (uint8_t*)codes, xscale, z_debug, s_debug);
    return hipGetLastError();
}

template <typename Tin, int BITS, bool HAD, bool TILED>
hipError_t dispatch_k(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                      float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    switch (K) {
        case 256: return launch_one<8, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 512: return launch_one<9, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 1024: return launch_one<10, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 2048: return launch_one<11, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 4096: return launch_one<12, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 8192: return launch_one<13, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 16384: return launch_one<14, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 32768: return launch_one<15, Tin, BITS, HAD, TILED>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tin, bool TILED>
hipError_t dispatch_mode(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                         float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    if (cfg.act_bits == 8) {
        return cfg.hadamard ? dispatch_k<Tin, 8, true, TILED>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                            : dispatch_k<Tin, 8, false, TILED>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    }
    return cfg.hadamard ? dispatch_k<Tin, 4, true, TILED>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                        : dispatch_k<Tin, 4, false, TILED>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

}  // namespace

hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                            const hbl_config& cfg, void* codes, float* xscale, float* z_debug, float* s_debug,
                            hipStream_t s, bool dec_tiled) {
    if (M == 0) return hipSuccess;
    if (dec_tiled) {
        if (x_dtype == HBL_F32)
            return dispatch_mode<float, true>((const float*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
        return dispatch_mode<uint16_t, true>((const uint16_t*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    }
    if (x_dtype == HBL_F32)
        return dispatch_mode<float, false>((const float*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    return dispatch_mode<uint16_t, false>((const uint16_t*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

}  // namespace hbl
