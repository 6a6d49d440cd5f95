// act_quant.hip -- fused per-token RMSNorm/LayerNorm + online fast Walsh-Hadamard
// transform + INT8/INT4 quantisation and packing (gfx950).
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块": the
// activations of H-BitLinear are normalised (LN in the layer formula; the
// architecture section "BitNet v2：原生4位激活" uses RMSNorm), rotated by an online
// Hadamard transform computed with a fast O(n log n) algorithm, then quantised
// per token to 8 or 4 bits.  The Hadamard is the normalised Sylvester matrix in
// natural order, H[i][j] = (-1)^popcount(i&j)/sqrt(K).
//
// One workgroup per token row.  Index bits of the row are processed as
// independent radix-2 butterfly stages (H_K is the Kronecker product of K's
// log2 factors H_2, so stage order is free):
//   1. vectorised 16-byte loads; thread t holds chunks c of V consecutive
//      elements at (c*NT + t)*V -- the V-bits and the chunk bits are in
//      registers, so those stages run before anything leaves the registers;
//   2. the row goes to LDS (fp32, one pad word per 32) and the remaining
//      log2(NT) "thread" bits are done in LDS passes of up to log2(E) bits
//      (E = K/NT values per thread);
//   3. each thread reads back Q consecutive values per chunk, forms the
//      per-token statistic (max|z| exactly, or sum|z| in fp64), and writes
//      packed codes with 16-byte stores.
// The norm scale is a per-row scalar, so it is applied before the transform
// (H(c r) = c H(r)); a gain vector, when given, multiplies x at load time.
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

HBL_DEVINL int pad_idx(int i) { return i + (i >> 5); }

template <typename T>
struct In;
template <>
struct In<float> {
    static constexpr int vec = 4;  // elements per 16-byte load
    template <int V>
    static HBL_DEVINL void load(const float* p, float* v) {
        if constexpr (V == 4) {
            const float4 q = *reinterpret_cast<const float4*>(p);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else if constexpr (V == 2) {
            const float2 q = *reinterpret_cast<const float2*>(p);
            v[0] = q.x; v[1] = q.y;
        } else {
#pragma unroll
            for (int j = 0; j < V; j++) v[j] = p[j];
        }
    }
};
template <>
struct In<uint16_t> {
    static constexpr int vec = 8;
    template <int V>
    static HBL_DEVINL void load(const uint16_t* p, float* v) {
        if constexpr (V == 8) {
            const uint4 q = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
        } else if constexpr (V == 4) {
            const uint2 q = *reinterpret_cast<const uint2*>(p);
            v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        } else {
#pragma unroll
            for (int j = 0; j < V; j++) v[j] = __uint_as_float(((uint32_t)p[j]) << 16);
        }
    }
};

// Radix-2 butterflies over every register bit of an E-element array.
template <int E>
HBL_DEVINL void reg_fwht(float* v) {
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int j = 0; j < E; j++) {
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

// Butterflies over index bits [LO, LO+R) through LDS: each thread takes
// E / 2^R groups of 2^R values spaced 2^LO apart.
template <int LK, int NT, int E, int LO, int R>
HBL_DEVINL void lds_pass(float* lds) {
    constexpr int G = E >> R;
    constexpr int S = 1 << R;
    float v[E];
#pragma unroll
    for (int g = 0; g < G; g++) {
        const int gam = g * NT + threadIdx.x;
        const int base = (gam & ((1 << LO) - 1)) | ((gam >> LO) << (LO + R));
#pragma unroll
        for (int j = 0; j < S; j++) v[g * S + j] = lds[pad_idx(base + (j << LO))];
    }
#pragma unroll
    for (int g = 0; g < G; g++) reg_fwht<S>(v + g * S);
#pragma unroll
    for (int g = 0; g < G; g++) {
        const int gam = g * NT + threadIdx.x;
        const int base = (gam & ((1 << LO) - 1)) | ((gam >> LO) << (LO + R));
#pragma unroll
        for (int j = 0; j < S; j++) lds[pad_idx(base + (j << LO))] = v[g * S + j];
    }
    __syncthreads();
}

template <int LK, int NT, int E, int LO, int HI>
HBL_DEVINL void lds_passes(float* lds) {
    if constexpr (LO < HI) {
        constexpr int R = cmin(ilog2(E), HI - LO);
        lds_pass<LK, NT, E, LO, R>(lds);
        lds_passes<LK, NT, E, LO + R, HI>(lds);
    }
}

template <int BITS>
HBL_DEVINL int quant1(float z, float s) {
    constexpr float lo = BITS == 8 ? -128.f : -8.f;
    constexpr float hi = BITS == 8 ? 127.f : 7.f;
    const float t = z * s;  // one rounded fp32 product
    return (int)fminf(fmaxf(rintf(t), lo), hi);
}

template <int LK, int NT, typename Tin, int BITS, bool HAD>
__global__ __launch_bounds__(NT) void act_quant_kernel(const Tin* __restrict__ X, const float* __restrict__ gain,
                                                       int norm, float norm_eps, float quant_eps, int a4_mode,
                                                       uint8_t* __restrict__ codes, float* __restrict__ xscale,
                                                       float* __restrict__ z_debug, float* __restrict__ s_debug) {
    constexpr int K = 1 << LK;
    constexpr int LT = ilog2(NT);
    constexpr int E = K / NT;
    static_assert(E >= 1 && (E & (E - 1)) == 0, "E must be a power of two");
    constexpr int V = cmin(In<Tin>::vec, E);
    constexpr int LV = ilog2(V);
    constexpr int C = E / V;
    constexpr int Q = cmin(E, BITS == 8 ? 16 : 32);  // values per store chunk
    constexpr int CQ = E / Q;

    extern __shared__ float lds[];
    __shared__ float redf[NT / kWave];
    __shared__ double redd[NT / kWave];

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const Tin* x = X + row * K;

    // ---- 1. load (chunk c holds elements (c*NT + tid)*V .. +V-1)
    float v[E];
#pragma unroll
    for (int c = 0; c < C; c++) In<Tin>::template load<V>(x + (c * NT + tid) * V, v + c * V);

    // ---- norm statistics (per row scalars)
    float mu = 0.f, scale = 1.f;
    if (norm == HBL_NORM_LN) {
        float s1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) s1 += v[e];
        mu = block_sum_f32<NT>(s1, redf) / (float)K;
    }
    if (norm != HBL_NORM_NONE) {
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) {
            const float c = v[e] - mu;
            s2 += c * c;
        }
        const float var = block_sum_f32<NT>(s2, redf) / (float)K;
        scale = 1.f / sqrtf(var + norm_eps);
    }
    // the butterflies compute the unnormalised transform; 1/sqrt(K) joins the row scale
    if constexpr (HAD) scale *= 1.f / sqrtf((float)K);
    if (gain != nullptr) {
#pragma unroll
        for (int c = 0; c < C; c++)
#pragma unroll
            for (int j = 0; j < V; j++) v[c * V + j] = (v[c * V + j] - mu) * gain[(c * NT + tid) * V + j] * scale;
    } else {
#pragma unroll
        for (int e = 0; e < E; e++) v[e] = (v[e] - mu) * scale;
    }

    // ---- 2. Hadamard: register bits now, thread bits through LDS
    if constexpr (HAD) reg_fwht<E>(v);
#pragma unroll
    for (int c = 0; c < C; c++)
#pragma unroll
        for (int j = 0; j < V; j++) lds[pad_idx((c * NT + tid) * V + j)] = v[c * V + j];
    __syncthreads();
    if constexpr (HAD) lds_passes<LK, NT, E, LV, LV + LT>(lds);

    // ---- 3. store layout: chunk c holds elements (c*NT + tid)*Q .. +Q-1
#pragma unroll
    for (int c = 0; c < CQ; c++)
#pragma unroll
        for (int j = 0; j < Q; j++) v[c * Q + j] = lds[pad_idx((c * NT + tid) * Q + j)];

    float s_mul, d_out;
    if (BITS == 8 || a4_mode == HBL_A4_ABSMAX_7) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) m = fmaxf(m, fabsf(v[e]));
        const float gamma = block_max_f32<NT>(m, redf);
        const float num = BITS == 8 ? 127.f : 7.f;
        s_mul = gamma == 0.f ? 0.f : num / (gamma + quant_eps);
        d_out = gamma == 0.f ? 0.f : gamma / num;
    } else {
        double sa = 0.0;
#pragma unroll
        for (int e = 0; e < E; e++) sa += (double)fabsf(v[e]);
        const float beta = (float)(block_sum_f64<NT>(sa, redd) / (double)K);
        s_mul = beta == 0.f ? 0.f : sqrt7_f32() / (beta + quant_eps);
        d_out = beta == 0.f ? 0.f : beta / sqrt7_f32();
    }
    if (tid == 0) {
        xscale[row] = d_out;
        if (s_debug) s_debug[row] = s_mul;
    }
    if (z_debug) {
#pragma unroll
        for (int c = 0; c < CQ; c++)
#pragma unroll
            for (int j = 0; j < Q; j++) z_debug[row * K + (c * NT + tid) * Q + j] = v[c * Q + j];
    }

    if constexpr (BITS == 8) {
        int8_t* out = reinterpret_cast<int8_t*>(codes) + row * K;
#pragma unroll
        for (int c = 0; c < CQ; c++) {
            uint32_t w[Q / 4 > 0 ? Q / 4 : 1];
#pragma unroll
            for (int d = 0; d < Q / 4; d++) {
                uint32_t acc = 0;
#pragma unroll
                for (int b = 0; b < 4; b++) acc |= ((uint32_t)quant1<8>(v[c * Q + 4 * d + b], s_mul) & 0xFFu) << (8 * b);
                w[d] = acc;
            }
            int8_t* dst = out + (c * NT + tid) * Q;
            if constexpr (Q == 16) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            } else if constexpr (Q >= 4) {
#pragma unroll
                for (int d = 0; d < Q / 4; d++) reinterpret_cast<uint32_t*>(dst)[d] = w[d];
            } else {
#pragma unroll
                for (int j = 0; j < Q; j++) dst[j] = (int8_t)quant1<8>(v[c * Q + j], s_mul);
            }
        }
    } else {
        uint8_t* out = codes + row * (K / 2);
#pragma unroll
        for (int c = 0; c < CQ; c++) {
            constexpr int ND = Q / 8 > 0 ? Q / 8 : 1;
            uint32_t w[ND];
            if constexpr (Q >= 8) {
#pragma unroll
                for (int d = 0; d < Q / 8; d++) {
                    uint32_t acc = 0;
#pragma unroll
                    for (int b = 0; b < 8; b++)
                        acc |= ((uint32_t)quant1<4>(v[c * Q + 8 * d + b], s_mul) & 0xFu) << (4 * b);
                    w[d] = acc;
                }
            }
            uint8_t* dst = out + (c * NT + tid) * (Q / 2);
            if constexpr (Q == 32) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            } else if constexpr (Q >= 8) {
#pragma unroll
                for (int d = 0; d < Q / 8; d++) reinterpret_cast<uint32_t*>(dst)[d] = w[d];
            } else {
#pragma unroll
                for (int j = 0; j < Q / 2; j++) {
                    const uint32_t lo = (uint32_t)quant1<4>(v[c * Q + 2 * j], s_mul) & 0xFu;
                    const uint32_t hi = (uint32_t)quant1<4>(v[c * Q + 2 * j + 1], s_mul) & 0xFu;
                    dst[j] = (uint8_t)(lo | (hi << 4));
                }
            }
        }
    }
}

// Threads per row: E = K/NT values per thread, between 4 and 64.
constexpr int threads_for(int LK) {
    return LK <= 8 ? 64 : (LK <= 11 ? 64 : (LK == 12 ? 128 : 256));
}

template <int LK, typename Tin, int BITS, bool HAD>
hipError_t launch_one(const Tin* X, int64_t M, const float* gain, const hbl_config& cfg, void* codes, float* xscale,
                      float* z_debug, float* s_debug, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    constexpr int K = 1 << LK;
    const size_t lds_bytes = (size_t)(K + K / 32 + 1) * sizeof(float);
    auto kern = act_quant_kernel<LK, NT, Tin, BITS, HAD>;
    static bool attr_set = false;  // one attribute call per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // one workgroup per row; gridDim.x is limited to 2^31-1
    hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(NT), lds_bytes, s, X, gain, cfg.norm, cfg.norm_eps,
                       cfg.quant_eps, cfg.a4_mode, (uint8_t*)codes, xscale, z_debug, s_debug);
    return hipGetLastError();
}

template <typename Tin, int BITS, bool HAD>
hipError_t dispatch_k(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                      float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    switch (K) {
        case 64: return launch_one<6, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 128: return launch_one<7, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 256: return launch_one<8, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 512: return launch_one<9, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 1024: return launch_one<10, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 2048: return launch_one<11, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 4096: return launch_one<12, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 8192: return launch_one<13, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 16384: return launch_one<14, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        case 32768: return launch_one<15, Tin, BITS, HAD>(X, M, gain, cfg, codes, xscale, z_debug, s_debug, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename Tin>
hipError_t dispatch_mode(const Tin* X, int64_t M, int64_t K, const float* gain, const hbl_config& cfg, void* codes,
                         float* xscale, float* z_debug, float* s_debug, hipStream_t s) {
    if (cfg.act_bits == 8) {
        return cfg.hadamard ? dispatch_k<Tin, 8, true>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                            : dispatch_k<Tin, 8, false>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    }
    return cfg.hadamard ? dispatch_k<Tin, 4, true>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s)
                        : dispatch_k<Tin, 4, false>(X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

}  // namespace

hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                            const hbl_config& cfg, void* codes, float* xscale, float* z_debug, float* s_debug,
                            hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (x_dtype == HBL_F32)
        return dispatch_mode<float>((const float*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
    return dispatch_mode<uint16_t>((const uint16_t*)X, M, K, gain, cfg, codes, xscale, z_debug, s_debug, s);
}

}  // namespace hbl
