// act_row.h -- one token row of the fused per-token RMSNorm/LayerNorm + online
// fast Walsh-Hadamard transform + INT8/INT4 quantisation and packing (gfx950),
// as device routines for a workgroup of NT threads.  Internal header.
//
// Follows the "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块": the
// activations of H-BitLinear are normalised (LN in the layer formula; the
// architecture section "BitNet v2：原生4位激活" uses RMSNorm), rotated by an online
// Hadamard transform computed with a fast O(n log n) algorithm, then quantised
// per token to 8 or 4 bits.  The Hadamard is the normalised Sylvester matrix in
// natural order, H[i][j] = (-1)^popcount(i&j)/sqrt(K).
//
// One workgroup per token row, E = K/NT values per thread.  H_K is the
// Kronecker product of log2(K) copies of H_2, so its radix-2 butterfly stages
// (one per index bit) commute and can run in any order:
//   1. 16-byte vector loads: thread t holds chunks c of V consecutive elements
//      at (c*NT + t)*V.  The butterflies over those "register" index bits run
//      at once.
//   2. The remaining log2(NT) "thread" bits go through LDS in phases.  In every
//      phase the two lowest index bits stay inside a thread (so every LDS
//      access is a float4) and up to log2(E)-2 thread bits become register
//      bits.  LDS holds the fp32 row with one pad float4 per eight (at most
//      2-way bank conflicts for the access patterns used).
//   3. The last phase keeps its values in registers: the per-token statistic,
//      quantisation and code stores run from that layout (no extra LDS trip).
// The norm is a per-row scalar c = 1/sqrt(mean + eps), so by linearity it is
// applied after the transform together with 1/sqrt(K); its partial sums ride
// along with the first LDS barrier.  LayerNorm without a gain uses
// H(x - mu*1) = H(x) - mu*K*e_0 for the unnormalised butterflies (the first
// Sylvester row is all ones);
// LayerNorm with a gain centres and scales the inputs before the transform.
// Rounding uses the 1.5*2^23 trick (exactly round-half-to-even after the clamp).
#pragma once
#include "hbl_device.h"

namespace hbl {
namespace {

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
typedef float v16f_cvt __attribute__((ext_vector_type(16)));    // operand of the BF6 conversion
typedef unsigned v6u_cvt __attribute__((ext_vector_type(6)));   // its 32 packed 6-bit fields
constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

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

// Radix-2 butterflies over every bit of an S-element register array.
template <int S>
HBL_DEVINL void reg_fwht(float* v) {
#pragma unroll
    for (int h = 1; h < S; h <<= 1) {
#pragma unroll
        for (int j = 0; j < S; j++) {
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

// LDS float offset of the VW-vector that starts at element e (one pad vector per 8).
template <int VW>
HBL_DEVINL int lds_off(int e) {
    const int q = e / VW;
    return (q + (q >> 3)) * VW;
}

// Register layout of an LDS phase whose butterflies cover index bits [LO, LO+R):
// register j = (g*2^R + f)*VW + v holds element base(g, f) + v with
//   gamma = g*NT + tid, low part -> bits [VB, LO), high part -> bits [LO+R, LK),
//   f -> bits [LO, LO+R), v -> bits [0, VB).
// phase_elem gives base(g, f) for thread t.  With gamma = g*NT + t (t < NT) every
// bit of the result comes from either g, f or t, so base = elem(g, f, 0) |
// elem(0, 0, t) with disjoint bits, both multiples of VW, and lds_off splits
// the same way: the thread's part is computed once per phase and the (g, f)
// part is a constant of the unrolled loops (an immediate offset of the LDS
// access), not an address computation per access.
template <int NT, int VB, int LO, int R>
HBL_DEVINL int phase_elem(int g, int f, int t) {
    const int gam = g * NT + t;
    const int low = gam & ((1 << (LO - VB)) - 1);
    const int high = gam >> (LO - VB);
    return (low << VB) | (f << LO) | (high << (LO + R));
}
template <int NT, int VB, int LO, int R>
HBL_DEVINL int phase_base(int g, int f) {
    return phase_elem<NT, VB, LO, R>(0, 0, (int)threadIdx.x) + phase_elem<NT, VB, LO, R>(g, f, 0);
}

template <int NT, int E, int VB, int LO, int R>
HBL_DEVINL void phase_read(const float* lds, float* v) {
    constexpr int VW = 1 << VB, G = E >> (VB + R), S = 1 << R;
    const float* const base = lds + lds_off<VW>(phase_elem<NT, VB, LO, R>(0, 0, (int)threadIdx.x));
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
        for (int f = 0; f < S; f++) {
            const float* p = base + lds_off<VW>(phase_elem<NT, VB, LO, R>(g, f, 0));
            float* d = v + (g * S + f) * VW;
            if constexpr (VW == 4) {
                const float4 q = *reinterpret_cast<const float4*>(p);
                d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
            } else {
                const float2 q = *reinterpret_cast<const float2*>(p);
                d[0] = q.x; d[1] = q.y;
            }
        }
}

template <int NT, int E, int VB, int LO, int R>
HBL_DEVINL void phase_write(float* lds, const float* v) {
    constexpr int VW = 1 << VB, G = E >> (VB + R), S = 1 << R;
    float* const base = lds + lds_off<VW>(phase_elem<NT, VB, LO, R>(0, 0, (int)threadIdx.x));
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
        for (int f = 0; f < S; f++) {
            float* p = base + lds_off<VW>(phase_elem<NT, VB, LO, R>(g, f, 0));
            const float* s = v + (g * S + f) * VW;
            if constexpr (VW == 4) *reinterpret_cast<float4*>(p) = make_float4(s[0], s[1], s[2], s[3]);
            else *reinterpret_cast<float2*>(p) = make_float2(s[0], s[1]);
        }
}

// Butterflies over the f bits of each VW-vector group: elements (g, f, v) and
// (g, f ^ h, v) pair up for each f bit h.
template <int E, int VB, int R>
HBL_DEVINL void phase_fwht(float* v) {
    constexpr int VW = 1 << VB, S = 1 << R, G = E >> (VB + R);
#pragma unroll
    for (int g = 0; g < G; g++)
#pragma unroll
        for (int h = 1; h < S; h <<= 1)
#pragma unroll
            for (int f = 0; f < S; f++)
                if ((f & h) == 0)
#pragma unroll
                    for (int x = 0; x < VW; x++) {
                        float& a = v[(g * S + f) * VW + x];
                        float& b = v[(g * S + f + h) * VW + x];
                        const float s = a + b, d = a - b;
                        a = s;
                        b = d;
                    }
}

// The LDS phases for thread bits [LO, HI); the last one leaves its values in
// registers and reports its layout through LAST_LO / LAST_R.
template <int NT, int E, int VB, int FREE, int LO, int HI>
struct Phases {
    static constexpr int R = cmin(FREE, HI - LO);
    static constexpr bool last = LO + R >= HI;
    static constexpr int LAST_LO = last ? LO : Phases<NT, E, VB, FREE, LO + R, HI>::LAST_LO;
    static constexpr int LAST_R = last ? R : Phases<NT, E, VB, FREE, LO + R, HI>::LAST_R;
    static HBL_DEVINL void run(float* lds, float* v) {
        phase_read<NT, E, VB, LO, R>(lds, v);
        phase_fwht<E, VB, R>(v);
        if constexpr (!last) {
            phase_write<NT, E, VB, LO, R>(lds, v);
            __syncthreads();
            Phases<NT, E, VB, FREE, LO + R, HI>::run(lds, v);
        }
    }
};
template <int NT, int E, int VB, int FREE, int HI>
struct Phases<NT, E, VB, FREE, HI, HI> {
    static constexpr int LAST_LO = HI, LAST_R = 0;
    static HBL_DEVINL void run(float*, float*) {}
};

// code bits of a clamped value: t + 1.5*2^23 rounds t to the nearest integer,
// ties to even, and leaves it in the low mantissa bits (two's complement).
HBL_DEVINL uint32_t code_bits(float z, float s, float lo, float hi) {
    const float t = z * s;  // one rounded fp32 product
    return __float_as_uint(fminf(fmaxf(t, lo), hi) + 12582912.0f);
}
// The same where the clamp cannot bind; the product must still be rounded to
// fp32 before the add (no fused multiply-add).
HBL_DEVINL uint32_t code_bits_unclamped(float z, float s) {
#pragma clang fp contract(off)
    const float t = z * s;
    return __float_as_uint(t + 12582912.0f);
}

// Threads per row: E = K/NT values per thread (32 from K = 2048 to 16384).
constexpr int kActE = 32;
constexpr int threads_for(int LK) { return cmin(512, cmax(64, (1 << LK) / kActE)); }

// Compile-time shape of one row for NT threads.
template <int LK, int NT, typename Tin>
struct ActShape {
    static constexpr int K = 1 << LK;
    static constexpr int LT = ilog2(NT);
    static constexpr int E = K / NT;
    static constexpr int LE = ilog2(E);
    static_assert(E >= 4 && (E & (E - 1)) == 0, "need at least 4 values per thread");
    static constexpr int V = cmin(In<Tin>::vec, E);
    static constexpr int LV = ilog2(V);
    static constexpr int C = E / V;
    static constexpr int VB = LE >= 3 ? 2 : 1;  // index bits kept inside a thread in every LDS phase
    static constexpr int VW = 1 << VB;
    static constexpr int FREE = LE - VB;        // thread bits a phase can take into registers
    static constexpr int NW = NT / kWave;
    static constexpr int lds_floats = K + K / 8 + VW;  // padded fp32 row (Hadamard only)
};

// A thread's values of one row, and the block's reduction slots.
template <int LK, int NT, typename Tin>
using ActRegs = float[ActShape<LK, NT, Tin>::E];
template <int LK, int NT, typename Tin>
using ActPartF = float[2][ActShape<LK, NT, Tin>::NW];   // wave partials (fp32): sum of squares, max
template <int LK, int NT, typename Tin>
using ActPartD = double[3][ActShape<LK, NT, Tin>::NW];  // wave partials (fp64): LayerNorm sums, absmean

// Step 1: 16-byte vector loads (chunk c holds elements (c*NT + tid)*V .. +V-1).
template <int LK, int NT, typename Tin>
HBL_DEVINL void act_row_load(const Tin* __restrict__ x, ActRegs<LK, NT, Tin>& v) {
    using S = ActShape<LK, NT, Tin>;
    constexpr int V = S::V, C = S::C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < C; c++) In<Tin>::template load<V>(x + (c * NT + tid) * V, v + c * V);
}

// Steps 2-4 for the row whose values act_row_load put in v: norm, transform,
// statistic, codes.  crow receives the row's codes (K bytes INT8, K/2 INT4;
// global or LDS), *xs_out the dequant factor, z_row / s_out the optional
// parity outputs.  lds holds ActShape::lds_floats floats; partf / partd are
// the block's reduction slots.  Every thread of the block must call it.
// LAYOUT kCodesRowMajor: code byte kb of the row goes to crow + kb.
// kCodesDecTiled: crow is the row's base in the decode tile layout
// (dec_tile_row_base) and byte kb goes to crow + dec_tile_offset(kb).
// kCodesFp6 (INT4 only, four values per vector): the codes go out as FP6 E3M2
// in the FP6 GEMM layout (hbl_device.h): crow at the row's 96 bytes of K step
// 0, fp6_stride bytes between K steps, fp6_swz = the row's chunk swap.
template <int LK, int NT, typename Tin, int BITS, bool HAD, int LAYOUT = kCodesRowMajor>
HBL_DEVINL void act_row_quantise(ActRegs<LK, NT, Tin>& v, const float* __restrict__ gain, int norm, float norm_eps,
                                 float quant_eps, int a4_mode, float* lds, ActPartF<LK, NT, Tin>& partf,
                                 ActPartD<LK, NT, Tin>& partd, uint8_t* crow, float* xs_out, float* z_row,
                                 float* s_out, int64_t fp6_stride = 96, int fp6_swz = 0) {
    using S = ActShape<LK, NT, Tin>;
    constexpr int K = S::K, LT = S::LT, E = S::E, V = S::V, LV = S::LV, C = S::C, VB = S::VB, VW = S::VW;
    constexpr int FREE = S::FREE, NW = S::NW;
    using Ph = Phases<NT, E, VB, FREE, LV, LV + LT>;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;

    // Norm partial sums.  RMSNorm: sum x^2 in fp32 (relative error ~1e-7, far
    // inside the transform's tolerance).  LayerNorm without a gain: one pass
    // in fp64 (sum x and sum x^2, exact enough for large means).  LayerNorm
    // with a gain must centre and scale before the transform: two fp32 passes.
    const bool ln_gain = norm == HBL_NORM_LN && gain != nullptr;
    float mu_pre = 0.f;
    if (ln_gain) {
        float f1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) f1 += v[e];
        f1 = wave_sum_f32(f1);
        if (lane == 0) partf[0][wid] = f1;
        __syncthreads();
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) t += partf[0][w];
        mu_pre = t / (float)K;
        __syncthreads();
    }
    if (norm == HBL_NORM_RMS || ln_gain) {
        float f2 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) {
            const float c = v[e] - mu_pre;
            f2 += c * c;
        }
        f2 = wave_sum_f32(f2);
        if (lane == 0) partf[0][wid] = f2;
    } else if (norm == HBL_NORM_LN) {
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int e = 0; e < E; e++) {
            s1 += (double)v[e];
            s2 += (double)v[e] * (double)v[e];
        }
        s1 = wave_sum_f64(s1);
        s2 = wave_sum_f64(s2);
        if (lane == 0) { partd[0][wid] = s1; partd[1][wid] = s2; }
    }
    if (gain != nullptr) {
#pragma unroll
        for (int c = 0; c < C; c++)
#pragma unroll
            for (int j = 0; j < V; j++) v[c * V + j] = (v[c * V + j] - mu_pre) * gain[(c * NT + tid) * V + j];
    }

    // ---- 2. Hadamard: register bits now, thread bits through LDS
    if constexpr (HAD) {
        reg_fwht<E>(v);
        float* const base = lds + lds_off<VW>(tid * V);  // the thread's part of the offsets (see phase_elem)
#pragma unroll
        for (int c = 0; c < C; c++)
#pragma unroll
            for (int j = 0; j < V; j += VW) {
                float* p = base + lds_off<VW>(c * NT * V + j);
                if constexpr (VW == 4) *reinterpret_cast<float4*>(p) = make_float4(v[c * V + j], v[c * V + j + 1],
                                                                                   v[c * V + j + 2], v[c * V + j + 3]);
                else *reinterpret_cast<float2*>(p) = make_float2(v[c * V + j], v[c * V + j + 1]);
            }
    }
    __syncthreads();
    if constexpr (HAD) Ph::run(lds, v);

    // ---- row scalars: z = (y - mu*K*e0 [LN, no gain]) * c / sqrt(K)
    float scale = 1.f, mu = 0.f;
    if (norm == HBL_NORM_LN && !ln_gain) {
        double t1 = 0.0, t2 = 0.0;
#pragma unroll
        for (int w = 0; w < NW; w++) { t1 += partd[0][w]; t2 += partd[1][w]; }
        const double m = t1 / K;
        const double var = t2 / K - m * m;
        mu = (float)m;
        scale = 1.f / sqrtf((float)(var < 0.0 ? 0.0 : var) + norm_eps);
    } else if (norm != HBL_NORM_NONE) {
        float t2 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) t2 += partf[0][w];
        scale = 1.f / sqrtf(t2 / (float)K + norm_eps);
    }
    if constexpr (HAD) scale *= 1.f / sqrtf((float)K);
    // index 0 is register 0 of thread 0 in every layout used here
    if constexpr (HAD) {
        if (norm == HBL_NORM_LN && !ln_gain && tid == 0) v[0] -= mu * (float)K;  // unnormalised H*1 = K*e_0
    } else {
        if (norm == HBL_NORM_LN && !ln_gain) {
#pragma unroll
            for (int e = 0; e < E; e++) v[e] -= mu;
        }
    }
#pragma unroll
    for (int e = 0; e < E; e++) v[e] *= scale;

    // ---- 3. per-token statistic and quantiser scale
    float s_mul, d_out;
    if (BITS == 8 || a4_mode == HBL_A4_ABSMAX_7) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) m = fmaxf(m, fabsf(v[e]));
        m = wave_max_f32(m);
        if (lane == 0) partf[1][wid] = m;
        __syncthreads();
        float gamma = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) gamma = fmaxf(gamma, partf[1][w]);
        const float num = BITS == 8 ? 127.f : 7.f;
        s_mul = gamma == 0.f ? 0.f : num / (gamma + quant_eps);
        d_out = gamma == 0.f ? 0.f : gamma / num;
    } else {
        // fp64 sum of |z|: the scale then matches the oracle's fp64 mean
        double sa = 0.0;
#pragma unroll
        for (int e = 0; e < E; e++) sa += (double)fabsf(v[e]);
        sa = wave_sum_f64(sa);
        if (lane == 0) partd[2][wid] = sa;
        __syncthreads();
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < NW; w++) t += partd[2][w];
        const float beta = (float)(t / (double)K);
        s_mul = beta == 0.f ? 0.f : sqrt7_f32() / (beta + quant_eps);
        d_out = beta == 0.f ? 0.f : beta / sqrt7_f32();
    }
    // With quant_eps = 0 a statistic below num / FLT_MAX (a row of magnitude
    // about 1e-37 or less) overflows the multiplier to +inf; such a row is
    // taken as a zero statistic (s = d = 0, codes 0), as the oracle reads it.
    if (__builtin_isinf(s_mul)) {
        s_mul = 0.f;
        d_out = 0.f;
    }
    if (tid == 0) {
        *xs_out = d_out;
        if (s_out) *s_out = s_mul;
    }

    // ---- 4. codes, written from the current layout in VW-vectors
    constexpr float lo = BITS == 8 ? -128.f : -8.f;
    constexpr float hi = BITS == 8 ? 127.f : 7.f;
    constexpr int SLO = HAD ? Ph::LAST_LO : 0;
    constexpr int SR = HAD ? Ph::LAST_R : 0;
    constexpr int NVEC = E / VW;
    // FP6: the rounded codes as floats and each vector's element index, for
    // the conversion after the loop
    constexpr bool kFp6 = LAYOUT == kCodesFp6;
    float rq[kFp6 ? E : 1];
    int e0s[kFp6 ? NVEC : 1];
#pragma unroll
    for (int u = 0; u < NVEC; u++) {
        int e0;  // element index of vector u
        if constexpr (HAD) {
            e0 = phase_base<NT, VB, SLO, SR>(u >> SR, u & ((1 << SR) - 1));
        } else {
            const int j = u * VW;
            e0 = ((j / V) * NT + tid) * V + (j % V);
        }
        const float* z = v + u * VW;
        if (z_row) {
            float* zd = z_row + e0;
            if constexpr (VW == 4) *reinterpret_cast<float4*>(zd) = make_float4(z[0], z[1], z[2], z[3]);
            else *reinterpret_cast<float2*>(zd) = make_float2(z[0], z[1]);
        }
        if constexpr (kFp6) {
            static_assert(BITS == 4 && VW == 4, "FP6 codes: INT4 values, four per vector");
            // the same decision as code_bits: one rounded fp32 product, the
            // clamp, round half to even; the integer stays a float (+0 turns
            // a rounded -0 into +0, so code 0 is always the all-zero field)
#pragma unroll
            for (int x2 = 0; x2 < VW; x2++) {
                const float t = z[x2] * s_mul;
                rq[u * VW + x2] = __builtin_rintf(fminf(fmaxf(t, lo), hi)) + 0.0f;
            }
            e0s[u] = e0;
            continue;
        }
        uint32_t b[VW];
#pragma unroll
        for (int x2 = 0; x2 < VW; x2++) {
            // INT8: |z| <= gamma and s = 127/(gamma+eps) keep |z*s| <= 127 (at
            // most one rounding above it, which still rounds to 127), so the
            // clamp cannot bind and is skipped
            if constexpr (BITS == 8) b[x2] = code_bits_unclamped(z[x2], s_mul);
            else b[x2] = code_bits(z[x2], s_mul, lo, hi);
        }
        // a vector's 2 or 4 code bytes never cross a 16-byte chunk of the tile layout
        const int kb = BITS == 8 ? e0 : e0 / 2;
        uint8_t* const cdst = crow + (LAYOUT == kCodesDecTiled ? dec_tile_offset<BITS>(kb) : kb);
        if constexpr (BITS == 8) {
            if constexpr (VW == 4) {
                const uint32_t w01 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);  // [b0.0, b1.0, 0, 0]
                const uint32_t w23 = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);  // [0, 0, b2.0, b3.0]
                *reinterpret_cast<uint32_t*>(cdst) = w01 | w23;
            } else {
                *reinterpret_cast<uint16_t*>(cdst) =
                    (uint16_t)((b[0] & 0xFFu) | ((b[1] & 0xFFu) << 8));
            }
        } else {
            if constexpr (VW == 4) {
                const uint32_t lo2 = (b[0] & 0xFu) | ((b[1] & 0xFu) << 4);
                const uint32_t hi2 = (b[2] & 0xFu) | ((b[3] & 0xFu) << 4);
                *reinterpret_cast<uint16_t*>(cdst) = (uint16_t)(lo2 | (hi2 << 8));
            } else {
                *cdst = (uint8_t)((b[0] & 0xFu) | ((b[1] & 0xFu) << 4));
            }
        }
    }
    if constexpr (kFp6) {
        // The hardware conversion turns 32 floats into their BF6 (E3M2)
        // fields, field 2k from the first operand's element k and field
        // 2k + 1 from the second's; every code in [-8, 7] is exact and the
        // scale is 1.  Fed the even and the odd codes, it returns this
        // thread's 32 codes as one natural-order bit string of six dwords, in
        // which vector u's four fields are bits 24u .. 24u + 23.  Each
        // vector's 24 bits go to LDS as one dword at dword e0/4 (LDS is free
        // since the statistic's barrier), natural order.
        constexpr int NG = (E + 31) / 32;
#pragma unroll
        for (int g = 0; g < NG; g++) {
            v16f_cvt ev, od;
#pragma unroll
            for (int k = 0; k < 16; k++) {
                ev[k] = 32 * g + 2 * k < E ? rq[32 * g + 2 * k] : 0.f;
                od[k] = 32 * g + 2 * k + 1 < E ? rq[32 * g + 2 * k + 1] : 0.f;
            }
            const v6u_cvt f = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
#pragma unroll
            for (int uu = 0; uu < 8; uu++) {
                const int u = 8 * g + uu;
                if (u >= NVEC) break;
                const int bit = 24 * uu, d = bit >> 5, sh = bit & 31;
                uint32_t w;
                if (sh == 0) w = f[d];
                else if (d == 5) w = f[d] >> sh;
                else w = __builtin_amdgcn_alignbit(f[d + 1], f[d], sh);
                reinterpret_cast<uint32_t*>(lds)[e0s[u] / 4] = w & 0xFFFFFFu;
            }
        }
        // Each group of 16 codes (four staged dwords) becomes the 12 bytes of
        // its natural FP6 bit string and goes straight to its place in the
        // GEMM layout: per K step of 128 codes (8 groups, 96 bytes) operand
        // op = group/2 keeps its first 16 bytes in chunk op and its last 8 in
        // half op / 2 of chunk 4 + op % 2 (chunks swapped as fp6_swz says);
        // an even group fills bytes 0..11 of the operand, an odd one bytes
        // 12..23 (4 in the first piece, 8 in the second).  All stores 4-byte
        // aligned.
        __syncthreads();
        const uint4* src = reinterpret_cast<const uint4*>(lds);
        for (int q = tid; q < K / 16; q += NT) {
            const uint4 d = src[q];
            const uint32_t w0 = d.x | (d.y << 24), w1 = (d.y >> 8) | (d.z << 16), w2 = (d.z >> 16) | (d.w << 8);
            const int j = q & 7, op = j >> 1;
            uint8_t* const step = crow + fp6_stride * (q >> 3);
            uint8_t* const c16 = step + 16 * (op ^ fp6_swz);
            if ((j & 1) == 0) {
                uint32_t* p = reinterpret_cast<uint32_t*>(c16);
                p[0] = w0; p[1] = w1; p[2] = w2;
            } else {
                *reinterpret_cast<uint32_t*>(c16 + 12) = w0;
                *reinterpret_cast<uint2*>(step + 16 * (4 + ((op & 1) ^ fp6_swz)) + 8 * (op >> 1)) = make_uint2(w1, w2);
            }
        }
    }
}

}  // namespace
}  // namespace hbl
