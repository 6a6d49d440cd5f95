// forward_small.hip -- the whole H-BitLinear forward for one token in one
// launch (gfx950): every block quantises the token row itself (norm, online
// Hadamard, per-token scale, codes; the row routine of act_row.h, the same
// code and thread count as the standalone activation kernel, so the codes
// and scale are bit-identical) and then runs the small-M GEMV of int_dot.h
// on its 16 output columns.
//
// A one-token layer is latency-bound: a separate activation launch costs a
// launch plus a serial chain of barriers for one row, and the GEMV waits for
// it.  Here the row's inputs are loaded, then the block's weight stream is
// issued, and the row is quantised while the weights are in flight.  The
// repeated activation work (one K-row per block, a few hundred vector
// operations per thread) is far below the weight-stream time.  For two or
// more tokens the rows would be quantised one after another in every block,
// which costs more than the separate launch; those go through the two stage
// kernels.
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块" (the
// layer: norm, online Hadamard, per-token quantisation, product with the
// ternary weights, rescale).
#include "act_row.h"
#include "int_dot.h"
#include "lds_attr.h"

namespace hbl {
namespace {

template <int LK, typename Tin, int BITS, bool HAD, typename YT>
__global__ __launch_bounds__(threads_for(LK)) void forward_small_kernel(
    const Tin* __restrict__ X, const float* __restrict__ gain, int norm, float norm_eps, float quant_eps,
    int a4_mode, const uint8_t* __restrict__ Wp, const float* __restrict__ alpha_p, int64_t N, YT* __restrict__ Y) {
    constexpr int NT = threads_for(LK);
    using S = ActShape<LK, NT, Tin>;
    using G = Gv<BITS, LK - 6, 1, NT>;
    extern __shared__ __attribute__((aligned(16))) float lds[];  // the fp32 row of the transform (float4 accesses)
    __shared__ ActPartF<LK, NT, Tin> partf;
    __shared__ ActPartD<LK, NT, Tin> partd;
    __shared__ __attribute__((aligned(16))) uint8_t codes_s[S::K * BITS / 8];
    __shared__ float xs_s[1];
    __shared__ typename G::Part part;
    const int64_t n0 = (int64_t)blockIdx.x * kGvRows;

    ActRegs<LK, NT, Tin> v;
    act_row_load<LK, NT, Tin>(X, v);    // the row first, then the weight stream
    __builtin_amdgcn_sched_barrier(0);  // keep every row load ahead of the weight loads
    typename G::WRegs w;
    G::load_w(Wp, n0, w);
    __builtin_amdgcn_sched_barrier(0);
    // straight-line code: the first use of v waits only for the row's own
    // (older) loads, not for the weight stream
    act_row_quantise<LK, NT, Tin, BITS, HAD>(v, gain, norm, norm_eps, quant_eps, a4_mode, lds, partf, partd, codes_s,
                                             xs_s, nullptr, nullptr);
    __syncthreads();
    typename G::ARegs a;
    G::load_codes_lds(codes_s, 1, a);
    typename G::AOps av;
    G::unpack_codes(a, av);
    typename G::Acc acc;
    G::dot(w, av, acc);
    G::template finish<YT>(acc, part, 1, xs_s, *alpha_p, N, Y, n0);
}

template <int LK, typename Tin, int BITS, bool HAD, typename YT>
hipError_t launch_fs(const Tin* X, const float* gain, const hbl_config& cfg, const uint8_t* Wp, const float* alpha,
                     int64_t N, YT* Y, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    const size_t lds_bytes = HAD ? (size_t)ActShape<LK, NT, Tin>::lds_floats * sizeof(float) : 0;
    auto kern = forward_small_kernel<LK, Tin, BITS, HAD, YT>;
    static std::atomic<uint32_t> lds_set{0};  // devices with the LDS limit raised for this kernel
    if (hipError_t e = set_dynamic_lds(kern, lds_bytes, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(N / kGvRows)), dim3(NT), lds_bytes, s, X, gain, cfg.norm, cfg.norm_eps,
                       cfg.quant_eps, cfg.a4_mode, Wp, alpha, N, Y);
    return hipGetLastError();
}

template <typename Tin, int BITS, bool HAD, typename YT>
hipError_t dispatch_k(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg,
                      const uint8_t* Wp, const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    switch (K) {
        case 1024: return launch_fs<10, Tin, BITS, HAD, YT>(X, gain, cfg, Wp, alpha, N, Y, s);
        case 2048: return launch_fs<11, Tin, BITS, HAD, YT>(X, gain, cfg, Wp, alpha, N, Y, s);
        case 4096: return launch_fs<12, Tin, BITS, HAD, YT>(X, gain, cfg, Wp, alpha, N, Y, s);
        case 8192: return launch_fs<13, Tin, BITS, HAD, YT>(X, gain, cfg, Wp, alpha, N, Y, s);
        case 16384: return launch_fs<14, Tin, BITS, HAD, YT>(X, gain, cfg, Wp, alpha, N, Y, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tin, typename YT>
hipError_t dispatch_mode(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg,
                         const uint8_t* Wp, const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    if (cfg.act_bits == 8)
        return cfg.hadamard ? dispatch_k<Tin, 8, true, YT>(X, M, K, gain, cfg, Wp, alpha, N, Y, s)
                            : dispatch_k<Tin, 8, false, YT>(X, M, K, gain, cfg, Wp, alpha, N, Y, s);
    return cfg.hadamard ? dispatch_k<Tin, 4, true, YT>(X, M, K, gain, cfg, Wp, alpha, N, Y, s)
                        : dispatch_k<Tin, 4, false, YT>(X, M, K, gain, cfg, Wp, alpha, N, Y, s);
}

}  // namespace

bool forward_small_eligible(int64_t M, int64_t K) {
    return M >= 1 && M <= kForwardSmallMaxM && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0;
}

hipError_t launch_forward_small(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                                const hbl_config& cfg, const uint8_t* W_packed, const float* alpha, int64_t N,
                                void* Y, int y_dtype, hipStream_t s) {
    if (x_dtype == HBL_F32) {
        return y_dtype == HBL_F32
                   ? dispatch_mode<float, float>((const float*)X, M, K, gain, cfg, W_packed, alpha, N, (float*)Y, s)
                   : dispatch_mode<float, uint16_t>((const float*)X, M, K, gain, cfg, W_packed, alpha, N,
                                                    (uint16_t*)Y, s);
    }
    return y_dtype == HBL_F32
               ? dispatch_mode<uint16_t, float>((const uint16_t*)X, M, K, gain, cfg, W_packed, alpha, N, (float*)Y, s)
               : dispatch_mode<uint16_t, uint16_t>((const uint16_t*)X, M, K, gain, cfg, W_packed, alpha, N,
                                                   (uint16_t*)Y, s);
}

}  // namespace hbl
