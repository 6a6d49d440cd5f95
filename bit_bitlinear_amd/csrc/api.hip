// api.hip -- the C ABI of libhbl.so: host-side validation, workspace carving
// and kernel dispatch.  Every argument is checked before anything is queued,
// so invalid calls return an error without touching the GPU.
#include <hip/hip_runtime.h>

#include "hbl.h"
#include "hbl_device.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

hbl_status hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return HBL_ERR_HIP;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool dtype_ok(int32_t d) { return d == HBL_F32 || d == HBL_BF16; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int64_t kMaxGemmM = int64_t(1) << 23;
constexpr int64_t kMaxGemmN = int64_t(1) << 20;  // keeps a 128-row output tile's byte offsets in 32 bits
// Activation quantisation and weight packing share a grid up to this row
// length; for longer rows (one workgroup of 128-512 threads per row, 17-147
// KiB of LDS) the shared grid measured no faster than two launches.
constexpr int64_t kFuseActPackMaxK = 2048;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
// The base-3 GEMV: one lane per 16-byte vector of a row (at most 256 of them)
// and the codes of up to four tokens in registers.
constexpr int64_t kMaxBase3M = 4, kMaxBase3K = 16384;

hbl_status check_weight_shape(int64_t N, int64_t K) {
    if (N < 1 || K < 16) return HBL_ERR_SHAPE;
    if (K % 16) return HBL_ERR_ALIGN;
    if (N > (int64_t(1) << 40) / K) return HBL_ERR_SHAPE;
    return HBL_OK;
}

hbl_status check_config(const hbl_config* cfg) {
    if (!cfg) return HBL_ERR_NULL;
    if (cfg->act_bits != 8 && cfg->act_bits != 4) return HBL_ERR_BITS;
    if (cfg->hadamard != 0 && cfg->hadamard != 1) return HBL_ERR_BITS;
    if (cfg->norm != HBL_NORM_RMS && cfg->norm != HBL_NORM_LN && cfg->norm != HBL_NORM_NONE) return HBL_ERR_BITS;
    if (cfg->act_bits == 4 && cfg->a4_mode != HBL_A4_ABSMEAN_SQRT7 && cfg->a4_mode != HBL_A4_ABSMAX_7)
        return HBL_ERR_BITS;
    if (!(cfg->norm_eps >= 0.f) || !(cfg->quant_eps >= 0.f)) return HBL_ERR_SHAPE;
    return HBL_OK;
}

hbl_status check_act_shape(int64_t M, int64_t K) {
    if (M < 0 || M > kMaxRows) return HBL_ERR_SHAPE;
    if (K < HBL_MIN_K || K > HBL_MAX_K) return HBL_ERR_SHAPE;
    if (!is_pow2(K)) return HBL_ERR_NOT_POW2;
    return HBL_OK;
}

hbl_status check_gemm_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || M > kMaxGemmM) return HBL_ERR_SHAPE;
    if (K < 128 || K > HBL_MAX_K) return HBL_ERR_SHAPE;
    if (K % 128) return HBL_ERR_ALIGN;
    if (N < 16 || N > kMaxGemmN) return HBL_ERR_SHAPE;
    if (N % 16) return HBL_ERR_ALIGN;
    return HBL_OK;
}

size_t codes_bytes(int64_t M, int64_t K, int32_t bits) { return (size_t)M * (size_t)K * (size_t)bits / 8; }

// Workspace of the FP6 x FP4 path: FP6 codes (K*3/4 bytes per row), the
// per-token scales, and the weights as FP4 (K/2 bytes per row).
size_t f6f4_ws_bytes(int64_t M, int64_t K, int64_t N) {
    return round_up((size_t)M * (size_t)K * 3 / 4, 256) + round_up((size_t)M * sizeof(float), 256) +
           round_up((size_t)N * (size_t)K / 2, 256);
}

// The forward takes the FP6 x FP4 GEMM for INT4 prefill shapes when the
// caller's workspace holds its larger layout (hbl_forward_workspace_bytes).
bool use_f6f4(int64_t M, int64_t K, int64_t N, const hbl_config* cfg, size_t ws_bytes) {
    return cfg->act_bits == 4 && hbl::gemm_f6f4_eligible(M, K, N) && ws_bytes >= f6f4_ws_bytes(M, K, N);
}

// Bytes of the codes region of the forward workspace: up to 64 rows it is
// padded to whole 16-row tiles, which the decode tile layout needs.
size_t ws_codes_bytes(int64_t M, int64_t K, int32_t bits) {
    return round_up(codes_bytes(M <= 64 ? (M + 15) / 16 * 16 : M, K, bits), 256);
}

}  // namespace

namespace hbl {
void record_hip_error(hipError_t e) { g_last_hip_error = (int32_t)e; }

hbl_status check_forward_args(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                              const uint8_t* W_packed, const float* alpha, int64_t N, const hbl_config* cfg,
                              const void* Y, int32_t y_dtype) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    if ((st = check_act_shape(M, K)) != HBL_OK) return st;
    if ((st = check_gemm_shape(M, K, N)) != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!X || !W_packed || !alpha || !Y) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(W_packed) || !aligned(alpha, 4) || !aligned16(Y) || !aligned(gain, 4))
        return HBL_ERR_ALIGN;
    return HBL_OK;
}
}  // namespace hbl

extern "C" {

const char* hbl_status_string(hbl_status s) {
    switch (s) {
        case HBL_OK: return "ok";
        case HBL_ERR_NULL: return "a required pointer is NULL";
        case HBL_ERR_SHAPE: return "a size is out of range";
        case HBL_ERR_NOT_POW2: return "K must be a power of two";
        case HBL_ERR_ALIGN: return "misaligned size or pointer (K, N multiples of 16; pointers 16-byte aligned)";
        case HBL_ERR_DTYPE: return "unknown dtype";
        case HBL_ERR_BITS: return "unsupported act_bits, a4_mode, norm or hadamard flag";
        case HBL_ERR_WORKSPACE: return "workspace too small";
        case HBL_ERR_UNSUPPORTED: return "request not supported by this library";
        case HBL_ERR_HIP: return "HIP error (see hbl_last_hip_error)";
    }
    return "unknown status";
}

int32_t hbl_last_hip_error(void) { return g_last_hip_error; }

hbl_status hbl_packed_weight_bytes(int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    *bytes = (size_t)N * (size_t)(K / 4);
    return HBL_OK;
}

hbl_status hbl_weight_workspace_bytes(int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    *bytes = (size_t)hbl::weight_partial_count(N * K) * sizeof(double);
    return HBL_OK;
}

hbl_status hbl_quantize_weights(const void* W, int32_t w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                                float* alpha, void* ws, size_t ws_bytes, void* stream) {
    if (!W || !W_packed || !alpha || !ws) return HBL_ERR_NULL;
    if (!dtype_ok(w_dtype)) return HBL_ERR_DTYPE;
    hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    if (!(eps >= 0.f)) return HBL_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned(alpha, 4) || !aligned(ws, 8)) return HBL_ERR_ALIGN;
    const int n_partial = hbl::weight_partial_count(N * K);
    if (ws_bytes < (size_t)n_partial * sizeof(double)) return HBL_ERR_WORKSPACE;
    hipError_t e = hbl::launch_weight_quant(W, w_dtype, N, K, eps, W_packed, alpha, (double*)ws, n_partial,
                                            (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_workspace_bytes(int64_t M, int64_t K, const hbl_config* cfg, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (M < 0 || M > kMaxRows || K < 1 || K > HBL_MAX_K) return HBL_ERR_SHAPE;
    *bytes = ws_codes_bytes(M, K, cfg->act_bits) + round_up((size_t)M * sizeof(float), 256);
    return HBL_OK;
}

hbl_status hbl_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, const hbl_config* cfg, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    hbl_status st = hbl_workspace_bytes(M, K, cfg, bytes);
    if (st != HBL_OK) return st;
    if (N < 1 || N > kMaxGemmN) return HBL_ERR_SHAPE;
    if (cfg->act_bits == 4 && hbl::gemm_f6f4_eligible(M, K, N)) {
        const size_t f = f6f4_ws_bytes(M, K, N);
        if (f > *bytes) *bytes = f;
    }
    return HBL_OK;
}

static hbl_status check_backward(int64_t M, int64_t K, int64_t N, const hbl_config* cfg) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if ((st = check_act_shape(M, K)) != HBL_OK) return st;
    if ((st = check_gemm_shape(M, K, N)) != HBL_OK) return st;
    if (K < 512) return HBL_ERR_SHAPE;                                     // four values per thread vector
    if (M > ((int64_t)1 << 21) || N > ((int64_t)1 << 21)) return HBL_ERR_SHAPE;  // tile offsets, grid sizes
    return HBL_OK;
}

hbl_status hbl_backward_workspace_bytes(int64_t M, int64_t K, int64_t N, const hbl_config* cfg, int32_t with_dw,
                                        size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    const hbl_status st = check_backward(M, K, N, cfg);
    if (st != HBL_OK) return st;
    *bytes = hbl::backward_ws_bytes(M, K, N, cfg->act_bits, with_dw != 0);
    return HBL_OK;
}

hbl_status hbl_backward(const void* dY, int32_t dy_dtype, const void* X, int32_t x_dtype, int64_t M, int64_t K,
                        const float* gain, const uint8_t* W_packed, const float* alpha, int64_t N,
                        const hbl_config* cfg, float* dX, float* dW, void* ws, size_t ws_bytes, void* stream) {
    hbl_status st = check_backward(M, K, N, cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(dy_dtype) || !dtype_ok(x_dtype)) return HBL_ERR_DTYPE;
    if (M == 0) return HBL_OK;
    if (!dY || !X || !W_packed || !alpha || !dX || !ws) return HBL_ERR_NULL;
    if (!aligned16(dY) || !aligned16(X) || !aligned16(W_packed) || !aligned(alpha, 4) || !aligned16(dX) ||
        !aligned16(dW) || !aligned16(ws) || !aligned(gain, 4))
        return HBL_ERR_ALIGN;
    if (ws_bytes < hbl::backward_ws_bytes(M, K, N, cfg->act_bits, dW != nullptr)) return HBL_ERR_WORKSPACE;
    const hipError_t e = hbl::launch_backward(dY, dy_dtype, X, x_dtype, M, K, gain, W_packed, alpha, N, *cfg, dX, dW,
                                              ws, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_quantize_heads(const void* X, int32_t x_dtype, int64_t M, int64_t H, int64_t D, int32_t bits,
                              float eps, uint8_t* codes, float* scales, void* stream) {
    if (!dtype_ok(x_dtype)) return HBL_ERR_DTYPE;
    if (bits != 3 && bits != 4 && bits != 8) return HBL_ERR_BITS;
    if (M < 0 || H < 1 || !(eps >= 0.f)) return HBL_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128 && D != 256) return HBL_ERR_SHAPE;
    if (M > ((int64_t)1 << 40) / (H * D)) return HBL_ERR_SHAPE;  // M*H*D < 2^40 elements
    if (M == 0) return HBL_OK;
    if (!X || !codes || !scales) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(codes) || !aligned(scales, 4)) return HBL_ERR_ALIGN;
    const hipError_t e = hbl::launch_head_quant(X, x_dtype, M * H, D, bits, eps, codes, scales, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_quantize_activations(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                                    const hbl_config* cfg, void* codes, float* xscale, float* z_debug,
                                    float* s_debug, void* stream) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype)) return HBL_ERR_DTYPE;
    st = check_act_shape(M, K);
    if (st != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!X || !codes || !xscale) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(codes) || !aligned(xscale, 4) || !aligned16(z_debug) || !aligned(s_debug, 4) ||
        !aligned(gain, 4))
        return HBL_ERR_ALIGN;
    hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes, xscale, z_debug, s_debug,
                                         (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_gemm(const void* codes, const float* xscale, int32_t act_bits, int64_t M, int64_t K,
                    const uint8_t* W_packed, const float* alpha, int64_t N, void* Y, int32_t y_dtype, void* stream) {
    if (act_bits != 8 && act_bits != 4) return HBL_ERR_BITS;
    if (!dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    hbl_status st = check_gemm_shape(M, K, N);
    if (st != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!codes || !xscale || !W_packed || !alpha || !Y) return HBL_ERR_NULL;
    if (!aligned16(codes) || !aligned(xscale, 4) || !aligned16(W_packed) || !aligned(alpha, 4) || !aligned16(Y))
        return HBL_ERR_ALIGN;
    hipError_t e = hbl::launch_gemm(codes, xscale, act_bits, M, K, W_packed, alpha, N, Y, y_dtype,
                                    (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_forward(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                       const uint8_t* W_packed, const float* alpha, int64_t N, const hbl_config* cfg, void* Y,
                       int32_t y_dtype, void* ws, size_t ws_bytes, void* stream) {
    hbl_status st = hbl::check_forward_args(X, x_dtype, M, K, gain, W_packed, alpha, N, cfg, Y, y_dtype);
    if (st != HBL_OK || M == 0) return st;
    if (!ws) return HBL_ERR_NULL;
    if (!aligned16(ws)) return HBL_ERR_ALIGN;
    const size_t cb = ws_codes_bytes(M, K, cfg->act_bits);
    const size_t need = cb + round_up((size_t)M * sizeof(float), 256);
    if (ws_bytes < need) return HBL_ERR_WORKSPACE;
    if (hbl::forward_small_eligible(M, K)) {
        const hipError_t e = hbl::launch_forward_small(X, x_dtype, M, K, gain, *cfg, W_packed, alpha, N, Y, y_dtype,
                                                       (hipStream_t)stream);
        return e == hipSuccess ? HBL_OK : hip_fail(e);
    }
    const hipStream_t s = (hipStream_t)stream;
    if (use_f6f4(M, K, N, cfg, ws_bytes)) {
        uint8_t* codes6 = (uint8_t*)ws;
        float* xs = (float*)(codes6 + round_up((size_t)M * (size_t)K * 3 / 4, 256));
        uint8_t* W4 = (uint8_t*)xs + round_up((size_t)M * sizeof(float), 256);
        hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes6, xs, nullptr, nullptr, s,
                                             hbl::kCodesFp6);
        if (e == hipSuccess) e = hbl::launch_weights_to_fp4(W_packed, N, K, W4, s);
        if (e == hipSuccess) e = hbl::launch_gemm_f6f4(codes6, xs, M, K, W4, alpha, N, Y, y_dtype, s);
        return e == hipSuccess ? HBL_OK : hip_fail(e);
    }
    void* codes = ws;
    float* xscale = (float*)((uint8_t*)ws + cb);
    // codes that only the decode GEMM reads go out in its tile layout
    const bool tiled = hbl::gemm_uses_decode_kernel(M, K);
    hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes, xscale, nullptr, nullptr, s,
                                         tiled ? hbl::kCodesDecTiled : hbl::kCodesRowMajor);
    if (e != hipSuccess) return hip_fail(e);
    e = hbl::launch_gemm(codes, xscale, cfg->act_bits, M, K, W_packed, alpha, N, Y, y_dtype, s, tiled);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_forward_latent(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain, const void* W,
                              int32_t w_dtype, int64_t N, float w_eps, const hbl_config* cfg, uint8_t* W_packed,
                              float* alpha, void* Y, int32_t y_dtype, void* ws, size_t ws_bytes, void* wws,
                              size_t wws_bytes, void* stream) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype) || !dtype_ok(w_dtype)) return HBL_ERR_DTYPE;
    if ((st = check_weight_shape(N, K)) != HBL_OK) return st;
    if ((st = check_act_shape(M, K)) != HBL_OK) return st;
    if ((st = check_gemm_shape(M, K, N)) != HBL_OK) return st;
    if (!(w_eps >= 0.f)) return HBL_ERR_SHAPE;
    if (!W || !W_packed || !alpha || !wws) return HBL_ERR_NULL;
    if (M > 0 && (!X || !Y || !ws)) return HBL_ERR_NULL;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned(alpha, 4) || !aligned(wws, 8)) return HBL_ERR_ALIGN;
    if (M > 0 && (!aligned16(X) || !aligned16(Y) || !aligned16(ws) || !aligned(gain, 4))) return HBL_ERR_ALIGN;
    const int n_partial = hbl::weight_partial_count(N * K);
    if (wws_bytes < (size_t)n_partial * sizeof(double)) return HBL_ERR_WORKSPACE;
    const size_t cb = ws_codes_bytes(M, K, cfg->act_bits);
    if (M > 0 && ws_bytes < cb + round_up((size_t)M * sizeof(float), 256)) return HBL_ERR_WORKSPACE;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (M == 0 || hbl::forward_small_eligible(M, K)) {
        // no rows, or one token whose whole forward is a single launch
        e = hbl::launch_weight_quant(W, w_dtype, N, K, w_eps, W_packed, alpha, (double*)wws, n_partial, s);
        if (e == hipSuccess && M > 0)
            e = hbl::launch_forward_small(X, x_dtype, M, K, gain, *cfg, W_packed, alpha, N, Y, y_dtype, s);
        return e == hipSuccess ? HBL_OK : hip_fail(e);
    }
    const bool f6 = use_f6f4(M, K, N, cfg, ws_bytes);
    void* codes = ws;
    float* xscale = (float*)((uint8_t*)ws + (f6 ? round_up((size_t)M * (size_t)K * 3 / 4, 256) : cb));
    uint8_t* W4 = (uint8_t*)xscale + round_up((size_t)M * sizeof(float), 256);  // FP6 x FP4 path only
    const bool tiled = hbl::gemm_uses_decode_kernel(M, K);
    const int layout = f6 ? hbl::kCodesFp6 : tiled ? hbl::kCodesDecTiled : hbl::kCodesRowMajor;
    if (K <= kFuseActPackMaxK) {
        // short rows: the activation rows share one grid with the partial |W|
        // sums (neither needs the other), then the packing
        e = hbl::launch_act_and_pack(X, x_dtype, M, K, gain, *cfg, codes, xscale, W, w_dtype, N * K, w_eps, nullptr,
                                     (double*)wws, n_partial, W_packed, alpha, s, layout);
        if (e == hipSuccess)
            e = hbl::launch_weight_pack(W, w_dtype, N, K, w_eps, W_packed, alpha, (const double*)wws, n_partial, s);
    } else {
        e = hbl::launch_weight_quant(W, w_dtype, N, K, w_eps, W_packed, alpha, (double*)wws, n_partial, s);
        if (e == hipSuccess)
            e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes, xscale, nullptr, nullptr, s, layout);
    }
    if (f6) {
        if (e == hipSuccess) e = hbl::launch_weights_to_fp4(W_packed, N, K, W4, s);
        if (e == hipSuccess)
            e = hbl::launch_gemm_f6f4((const uint8_t*)codes, xscale, M, K, W4, alpha, N, Y, y_dtype, s);
    } else if (e == hipSuccess) {
        e = hbl::launch_gemm(codes, xscale, cfg->act_bits, M, K, W_packed, alpha, N, Y, y_dtype, s, tiled);
    }
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

// ------------------------------------------------ FP4 weights, FP6 codes --
// The INT4 prefill path on the FP6 x FP4 matrix cores with the weights
// converted to FP4 once, ahead of the forward passes.

static hbl_status check_fp6_act(int64_t M, int64_t K, const hbl_config* cfg) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (cfg->act_bits != 4) return HBL_ERR_BITS;
    if ((st = check_act_shape(M, K)) != HBL_OK) return st;
    if (K < 512) return HBL_ERR_SHAPE;  // whole FP6 operand pieces per row
    return HBL_OK;
}

static hbl_status check_fp6_gemm(int64_t M, int64_t K, int64_t N) {
    hbl_status st = check_gemm_shape(M, K, N);
    if (st != HBL_OK) return st;
    if (K < 512) return HBL_ERR_SHAPE;
    return HBL_OK;
}

static size_t fp6_codes_bytes(int64_t M, int64_t K) { return (size_t)M * (size_t)K * 3 / 4; }

// The FP4 weight format holds whole GEMM K steps of 128 weights.
static hbl_status check_fp4_shape(int64_t N, int64_t K) {
    const hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    return K % 128 ? HBL_ERR_ALIGN : HBL_OK;
}

hbl_status hbl_fp4_weight_bytes(int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    const hbl_status st = check_fp4_shape(N, K);
    if (st != HBL_OK) return st;
    *bytes = (size_t)N * (size_t)(K / 2);
    return HBL_OK;
}

hbl_status hbl_pack_fp4(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W4, void* stream) {
    const hbl_status st = check_fp4_shape(N, K);
    if (st != HBL_OK) return st;
    if (!W_packed || !W4) return HBL_ERR_NULL;
    if (!aligned16(W_packed) || !aligned16(W4)) return HBL_ERR_ALIGN;
    const hipError_t e = hbl::launch_weights_to_fp4(W_packed, N, K, W4, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_fp6_codes_bytes(int64_t M, int64_t K, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    if (M < 0 || M > kMaxRows || K < 512 || K > HBL_MAX_K) return HBL_ERR_SHAPE;
    if (K % 128) return HBL_ERR_ALIGN;
    *bytes = fp6_codes_bytes(M, K);
    return HBL_OK;
}

hbl_status hbl_quantize_activations_fp6(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                                        const hbl_config* cfg, uint8_t* codes6, float* xscale, void* stream) {
    hbl_status st = check_fp6_act(M, K, cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype)) return HBL_ERR_DTYPE;
    if (M == 0) return HBL_OK;
    if (!X || !codes6 || !xscale) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(codes6) || !aligned(xscale, 4) || !aligned(gain, 4)) return HBL_ERR_ALIGN;
    const hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes6, xscale, nullptr, nullptr,
                                               (hipStream_t)stream, hbl::kCodesFp6);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_gemm_fp6fp4(const uint8_t* codes6, const float* xscale, int64_t M, int64_t K, const uint8_t* W4,
                           const float* alpha, int64_t N, void* Y, int32_t y_dtype, void* stream) {
    if (!dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    const hbl_status st = check_fp6_gemm(M, K, N);
    if (st != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!codes6 || !xscale || !W4 || !alpha || !Y) return HBL_ERR_NULL;
    if (!aligned16(codes6) || !aligned(xscale, 4) || !aligned16(W4) || !aligned(alpha, 4) || !aligned16(Y))
        return HBL_ERR_ALIGN;
    const hipError_t e = hbl::launch_gemm_f6f4(codes6, xscale, M, K, W4, alpha, N, Y, y_dtype, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_forward_fp4_workspace_bytes(int64_t M, int64_t K, const hbl_config* cfg, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    const hbl_status st = check_fp6_act(M, K, cfg);
    if (st != HBL_OK) return st;
    *bytes = round_up(fp6_codes_bytes(M, K), 256) + round_up((size_t)M * sizeof(float), 256);
    return HBL_OK;
}

hbl_status hbl_forward_fp4(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                           const uint8_t* W4, const float* alpha, int64_t N, const hbl_config* cfg, void* Y,
                           int32_t y_dtype, void* ws, size_t ws_bytes, void* stream) {
    hbl_status st = check_fp6_act(M, K, cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    if ((st = check_fp6_gemm(M, K, N)) != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!X || !W4 || !alpha || !Y || !ws) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(W4) || !aligned(alpha, 4) || !aligned16(Y) || !aligned16(ws) ||
        !aligned(gain, 4))
        return HBL_ERR_ALIGN;
    const size_t cb = round_up(fp6_codes_bytes(M, K), 256);
    if (ws_bytes < cb + round_up((size_t)M * sizeof(float), 256)) return HBL_ERR_WORKSPACE;
    const hipStream_t s = (hipStream_t)stream;
    uint8_t* codes6 = (uint8_t*)ws;
    float* xs = (float*)(codes6 + cb);
    hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, codes6, xs, nullptr, nullptr, s,
                                         hbl::kCodesFp6);
    if (e == hipSuccess) e = hbl::launch_gemm_f6f4(codes6, xs, M, K, W4, alpha, N, Y, y_dtype, s);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_base3_weight_bytes(int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return HBL_ERR_NULL;
    const hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    *bytes = (size_t)N * (size_t)hbl::base3_row_bytes(K);
    return HBL_OK;
}

hbl_status hbl_pack_base3(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W3, void* stream) {
    const hbl_status st = check_weight_shape(N, K);
    if (st != HBL_OK) return st;
    if (!W_packed || !W3) return HBL_ERR_NULL;
    if (!aligned16(W_packed) || !aligned16(W3)) return HBL_ERR_ALIGN;
    const hipError_t e = hbl::launch_pack_base3(W_packed, N, K, W3, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

static hbl_status check_base3_gemv_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || M > kMaxBase3M) return HBL_ERR_SHAPE;
    if (K < 16 || K > kMaxBase3K) return HBL_ERR_SHAPE;
    if (K % 16) return HBL_ERR_ALIGN;
    if (N < 1 || N > kMaxGemmN) return HBL_ERR_SHAPE;
    return HBL_OK;
}

hbl_status hbl_gemm_base3(const void* codes, const float* xscale, int32_t act_bits, int64_t M, int64_t K,
                          const uint8_t* W3, const float* alpha, int64_t N, void* Y, int32_t y_dtype, void* stream) {
    if (act_bits != 8 && act_bits != 4) return HBL_ERR_BITS;
    if (!dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    const hbl_status st = check_base3_gemv_shape(M, K, N);
    if (st != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!codes || !xscale || !W3 || !alpha || !Y) return HBL_ERR_NULL;
    if (!aligned16(codes) || !aligned(xscale, 4) || !aligned16(W3) || !aligned(alpha, 4) || !aligned16(Y))
        return HBL_ERR_ALIGN;
    const hipError_t e =
        hbl::launch_gemv_base3(codes, xscale, act_bits, M, K, W3, alpha, N, Y, y_dtype, (hipStream_t)stream);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

hbl_status hbl_forward_base3(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                             const uint8_t* W3, const float* alpha, int64_t N, const hbl_config* cfg, void* Y,
                             int32_t y_dtype, void* ws, size_t ws_bytes, void* stream) {
    hbl_status st = check_config(cfg);
    if (st != HBL_OK) return st;
    if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return HBL_ERR_DTYPE;
    st = check_act_shape(M, K);
    if (st != HBL_OK) return st;
    st = check_base3_gemv_shape(M, K, N);
    if (st != HBL_OK) return st;
    if (M == 0) return HBL_OK;
    if (!X || !W3 || !alpha || !Y || !ws) return HBL_ERR_NULL;
    if (!aligned16(X) || !aligned16(W3) || !aligned(alpha, 4) || !aligned16(Y) || !aligned16(ws) ||
        !aligned(gain, 4))
        return HBL_ERR_ALIGN;
    const size_t cb = ws_codes_bytes(M, K, cfg->act_bits);
    if (ws_bytes < cb + round_up((size_t)M * sizeof(float), 256)) return HBL_ERR_WORKSPACE;
    const hipStream_t s = (hipStream_t)stream;
    float* xscale = (float*)((uint8_t*)ws + cb);
    hipError_t e = hbl::launch_act_quant(X, x_dtype, M, K, gain, *cfg, ws, xscale, nullptr, nullptr, s);
    if (e == hipSuccess) e = hbl::launch_gemv_base3(ws, xscale, cfg->act_bits, M, K, W3, alpha, N, Y, y_dtype, s);
    return e == hipSuccess ? HBL_OK : hip_fail(e);
}

}  // extern "C"
