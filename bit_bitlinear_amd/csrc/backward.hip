// backward.hip -- the layer's backward with the straight-through estimator
// (gfx950): the quantisers are identities in the backward, so with
// y = alpha * d * (q . Wq^T):
//   dZ = alpha * dY . Wq           (bf16 matrix cores, fp32 sums)
//   dR = H dZ                      (the forward's fast transform: H is symmetric)
//   dX = norm'(x)^T dR             (RMSNorm / LayerNorm / none, with the gain)
//   dW = dY^T . (d * q)            (the forward's dequantised codes; bf16 matrix cores)
// Follows the xdnf.cn page "【AI论文】BitNet v2：针对1位LLM的原生4位激活和哈达玛
// 变换", section "研究方法" (training through the low-bit quantisers with a
// straight-through estimator), the 新智元 "微软 BitNet v2" repost, section
// "BitNet v2：原生4位激活" (training with low-bit activations and ternary
// weights), and its section "H-BitLinear模块" (the forward it differentiates).
//
// The two contractions are plain GEMMs on bf16 operands: the ternary weights
// and the integer codes are exact in bf16; dY (and dY * d for dW) is split
// into a bf16 high part and a bf16 remainder, so the operands carry about 16
// significant bits, and one launch runs the contraction over both parts
// (fp32 sums).  Operands are laid out "NT" (both with the contraction index
// contiguous, padded with zeros to a multiple of 64) by a split kernel and
// by converting transposes that widen to bf16 and transpose in one pass.
#include "act_row.h"
#include "lds_dma.h"
#include "lds_attr.h"

namespace hbl {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

HBL_DEVINL uint32_t bf16_bits_rne(float f) { return f32_to_bf16_bits(f); }

// ---------------------------------------------------------- operand prep ----
// v = in[r][c] * scale[r] (fp32 product; scale nullable) -> hi = bf16(v),
// lo = bf16(v - hi) (lo nullable), as [R][Cp] with zeros for c >= C; C and
// Cp multiples of 8; one thread per 8 consecutive elements of a row.
template <typename Tin>
__global__ __launch_bounds__(256) void split_bf16_kernel(const Tin* __restrict__ in, int64_t R, int64_t C,
                                                         int64_t Cp, const float* __restrict__ scale,
                                                         uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
    const int64_t c8 = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8, r = blockIdx.x;
    if (c8 >= Cp) return;
    float v[8];
    if (c8 < C) {
        const Tin* p = in + r * C + c8;
        if constexpr (sizeof(Tin) == 4) {
            const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            const uint4 q = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
        }
        if (scale) {
            const float sc = scale[r];
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = v[i] * sc;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = 0.f;
    }
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        h[i] = bf16_bits_rne(v[i]);
        l[i] = bf16_bits_rne(v[i] - __uint_as_float(h[i] << 16));
    }
    *reinterpret_cast<uint4*>(hi + r * Cp + c8) = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    if (lo)
        *reinterpret_cast<uint4*>(lo + r * Cp + c8) = make_uint4(l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16);
}

// ------------------------------------------- converting transposes ----
// out_o[c][r] = f_o(source)[r][c] for r < R (0 for R <= r < Rp), c < C: the
// conversion to bf16 and the transpose in one pass.  64 x 64 tiles, 256
// threads; each thread converts two runs of 8 consecutive c of one row (one
// 16-byte result each) into an LDS tile, then writes two runs of 8
// consecutive r of one output row as 16-byte stores.  C % 8 == 0, Rp % 64 == 0.
// Sources (load8 fills v[o][0..7] for (r, c .. c+7)):
//   TernSrc   2-bit weights [R][C/4] (R11 layout) -> 0, +1.0, -1.0
//   CodesSrc  INT8 [R][C] or INT4 [R][C/2] codes -> exact bf16 integers
//   SplitSrc  x = fp32(in[r][c] * scale[r]) -> bf16(x) and bf16(x - bf16(x))
struct TernSrc {
    static constexpr int NOUT = 1;
    const uint32_t* Wp;
    int64_t C;
    HBL_DEVINL void load8(int64_t r, int64_t c, uint32_t (&v)[2][8]) const {
        const uint32_t w = Wp[r * (C / 16) + c / 16];
        const int e0 = (int)(c & 15);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int e = e0 + j;
            const uint32_t code = (w >> (8 * (e & 3) + 2 * (e >> 2))) & 3u;
            v[0][j] = code == 1u ? 0x3F80u : code == 3u ? 0xBF80u : 0u;
        }
    }
};

template <int BITS>
struct CodesSrc {
    static constexpr int NOUT = 1;
    const uint8_t* codes;
    int64_t C;
    HBL_DEVINL void load8(int64_t r, int64_t c, uint32_t (&v)[2][8]) const {
        int q[8];
        if constexpr (BITS == 8) {
            const uint2 b = *reinterpret_cast<const uint2*>(codes + r * C + c);
#pragma unroll
            for (int e = 0; e < 4; e++) { q[e] = (int8_t)(b.x >> (8 * e)); q[4 + e] = (int8_t)(b.y >> (8 * e)); }
        } else {
            const uint32_t b = *reinterpret_cast<const uint32_t*>(codes + (r * C + c) / 2);
#pragma unroll
            for (int e = 0; e < 8; e++) q[e] = (int)(b << (28 - 4 * e)) >> 28;
        }
#pragma unroll
        for (int e = 0; e < 8; e++) v[0][e] = bf16_bits_rne((float)q[e]);  // exact: |q| <= 128
    }
};

template <typename Tin>
struct SplitSrc {
    static constexpr int NOUT = 2;
    const Tin* in;
    int64_t C;
    const float* scale;
    HBL_DEVINL void load8(int64_t r, int64_t c, uint32_t (&v)[2][8]) const {
        float x[8];
        const Tin* p = in + r * C + c;
        if constexpr (sizeof(Tin) == 4) {
            const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        } else {
            const uint4 q = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; i++) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
        }
        const float sc = scale[r];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float t = x[i] * sc;
            v[0][i] = bf16_bits_rne(t);
            v[1][i] = bf16_bits_rne(t - __uint_as_float(v[0][i] << 16));
        }
    }
};

constexpr int kCtRow = 72;  // LDS row stride in bf16 elements (144 bytes: 16-byte aligned, banks spread)

template <class Src>
__global__ __launch_bounds__(256) void convert_transpose_kernel(Src src, int64_t R, int64_t C, uint16_t* __restrict__ out0,
                                                                uint16_t* __restrict__ out1, int64_t Rp) {
    __shared__ __attribute__((aligned(16))) uint16_t t[Src::NOUT][64][kCtRow];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int idx = (int)threadIdx.x + 256 * i, rr = idx >> 3, cc = (idx & 7) * 8;
        const int64_t r = r0 + rr, c = c0 + cc;
        uint32_t v[2][8] = {};
        if (r < R && c < C) src.load8(r, c, v);
#pragma unroll
        for (int o = 0; o < Src::NOUT; o++)
            *reinterpret_cast<uint4*>(&t[o][rr][cc]) = make_uint4(v[o][0] | v[o][1] << 16, v[o][2] | v[o][3] << 16,
                                                                  v[o][4] | v[o][5] << 16, v[o][6] | v[o][7] << 16);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int idx = (int)threadIdx.x + 256 * i, cr = idx >> 3, rc = (idx & 7) * 8;
        const int64_t c = c0 + cr, r = r0 + rc;
        if (c < C && r < Rp) {
#pragma unroll
            for (int o = 0; o < Src::NOUT; o++) {
                uint32_t h[8];
#pragma unroll
                for (int j = 0; j < 8; j++) h[j] = t[o][rc + j][cr];
                *reinterpret_cast<uint4*>((o == 0 ? out0 : out1) + c * Rp + r) =
                    make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
            }
        }
    }
}

template <class Src>
void convert_transpose(const Src& src, int64_t R, int64_t C, uint16_t* out0, uint16_t* out1, int64_t Rp,
                       hipStream_t s) {
    hipLaunchKernelGGL((convert_transpose_kernel<Src>), dim3((unsigned)((C + 63) / 64), (unsigned)(Rp / 64)),
                       dim3(256), 0, s, src, R, C, out0, out1, Rp);
}

// ------------------------------------------------------------ bf16 GEMM ----
// C[r][s] = alpha * sum_t A[r][t] B[s][t], plus sum_t A2[r][t] B[s][t] when A2
// is given: the contraction then runs twice as long, its second half pairing
// A2 with the same B (the high part and the remainder of a split operand in
// one launch, so C is written once).  A, A2 [R][T], B [S][T] bf16 with
// T % 64 == 0 (zero padded), C fp32 [R][S].  Blocks of WGM x WGN waves, each
// a 64 x 64 wave tile (2 x 2 tiles of v_mfma_f32_32x32x16_bf16).  K step 64
// (128-byte operand rows): both tiles travel global -> LDS directly through a
// ring of S stages (the INT8 GEMM's loads, lds_dma.h), 16-byte chunk c of row
// r stored at c ^ ((r >> 1) & 7); MFMA step s of lane half h reads chunk
// 2s + h of its rows.
template <int WGM, int WGN, int S>
__global__ __launch_bounds__(64 * WGM * WGN, WGM * WGN == 4 ? 2 : 1) void gemm_bf16_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A2, const uint16_t* __restrict__ B, int64_t R,
    int64_t SN, int64_t T, float* __restrict__ C, const float* __restrict__ alpha_dev, float alpha_host) {
    constexpr int TA = 2, TB = 2, NW = WGM * WGN, BM = 64 * WGM, BN = 64 * WGN;
    constexpr int a_bytes = BM * 128, b_bytes = BN * 128, stage_bytes = a_bytes + b_bytes;
    constexpr int a_inst = a_bytes / 1024 / NW, b_inst = b_bytes / 1024 / NW, inst = a_inst + b_inst;
    static_assert(a_bytes % (1024 * NW) == 0 && b_bytes % (1024 * NW) == 0, "whole wave instructions");
    static_assert((S - 2) * inst < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * stage_bytes];
    const int64_t r0 = (int64_t)blockIdx.y * BM, s0 = (int64_t)blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t ld = T * 2;  // bytes per operand row
    const int KT1 = (int)(T / 64), KT = A2 ? 2 * KT1 : KT1;
    const v4u a_desc = rsrc_words(A + r0 * T, (R - r0) * ld);  // rows past R load as zeros
    const v4u a2_desc = rsrc_words((A2 ? A2 : A) + r0 * T, (R - r0) * ld);
    const v4u b_desc = rsrc_words(B + s0 * T, (SN - s0) * ld);
    uint32_t a_off[a_inst], b_off[b_inst];
#pragma unroll
    for (int u = 0; u < a_inst; u++) {
        const int c = (wave * a_inst + u) * 64 + lane, row = c >> 3, p = c & 7;
        a_off[u] = (uint32_t)(row * ld + ((p ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int u = 0; u < b_inst; u++) {
        const int c = (wave * b_inst + u) * 64 + lane, row = c >> 3, p = c & 7;
        b_off[u] = (uint32_t)(row * ld + ((p ^ ((row >> 1) & 7)) << 4));
    }
    const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    auto issue = [&](int kt, int st) {
        const uint32_t base = smem_addr + (uint32_t)(st * stage_bytes);
        const bool second = kt >= KT1;
        const uint32_t koff = (uint32_t)((second ? kt - KT1 : kt) * 128);
        const v4u ad = second ? a2_desc : a_desc;
#pragma unroll
        for (int u = 0; u < a_inst; u++)
            lds_dma16(ad, __builtin_amdgcn_readfirstlane(base + (uint32_t)((wave * a_inst + u) * 1024)), a_off[u] + koff);
#pragma unroll
        for (int u = 0; u < b_inst; u++)
            lds_dma16(b_desc, __builtin_amdgcn_readfirstlane(base + (uint32_t)(a_bytes + (wave * b_inst + u) * 1024)),
                      b_off[u] + koff);
    };
    v16f acc[TA][TB];
#pragma unroll
    for (int i = 0; i < TA; i++)
#pragma unroll
        for (int j = 0; j < TB; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    const int lr = lane & 31, lh = lane >> 5;
    auto frag = [&](const uint8_t* tile, int row, int ch) {
        return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(tile + row * 128 + ((ch ^ ((row >> 1) & 7)) << 4)));
    };
    auto compute = [&](int st) {
        const uint8_t* sa = smem + st * stage_bytes;
        const uint8_t* sb = sa + a_bytes;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            v8bf a[TA], b[TB];
#pragma unroll
            for (int i = 0; i < TA; i++) a[i] = frag(sa, wm * 32 * TA + i * 32 + lr, 2 * s + lh);
#pragma unroll
            for (int j = 0; j < TB; j++) b[j] = frag(sb, wn * 32 * TB + j * 32 + lr, 2 * s + lh);
#pragma unroll
            for (int i = 0; i < TA; i++)
#pragma unroll
                for (int j = 0; j < TB; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    // prologue: steps 0 .. S-2 in flight (past the last step the loads repeat
    // step KT-1, so every wave always has the same number in flight)
#pragma unroll
    for (int u = 0; u < S - 1; u++) issue(min(u, KT - 1), u);
    for (int kt = 0; kt < KT; kt++) {
        wait_vmcnt<(S - 2) * inst>();  // this wave's loads of step kt have landed
        barrier_no_wait();             // ... and every wave's; stage (kt-1)%S is free
        issue(min(kt + S - 1, KT - 1), (kt + S - 1) % S);
        compute(kt % S);
    }
    wait_vmcnt<0>();  // no LDS-direct load may still be in flight when the block ends
    const float alpha = alpha_dev ? *alpha_dev : alpha_host;
    // lane holds column lr of each 32 x 32 tile, rows 8*(r/4) + 4*lh + r%4
#pragma unroll
    for (int i = 0; i < TA; i++)
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int64_t sc = s0 + wn * 32 * TB + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = r0 + wm * 32 * TA + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < R && sc < SN) C[row * SN + sc] = alpha * acc[i][j][r];
            }
        }
}

template <int WGM, int WGN, int S>
hipError_t gemm_pair_shape(const uint16_t* A, const uint16_t* A2, const uint16_t* B, int64_t R, int64_t SN, int64_t T,
                           float* C, const float* alpha_dev, float alpha_host, hipStream_t s) {
    constexpr int BM = 64 * WGM, BN = 64 * WGN;
    const dim3 grid((unsigned)((SN + BN - 1) / BN), (unsigned)((R + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_bf16_dma_kernel<WGM, WGN, S>), grid, dim3(64 * WGM * WGN), 0, s, A, A2, B, R, SN, T, C,
                       alpha_dev, alpha_host);
    return hipGetLastError();
}

// 256 x 256 blocks of 16 waves once there are at least 256 of them (one per
// CU); 128 x 128 blocks of 4 waves (two per CU) below that.  Measured against
// 128 x 256 blocks of 8 waves, 64 x 128 wave tiles and three-stage rings,
// which were slower at both 4096 x 2048 x 2048 and 8192 x 16384 x 4096.
hipError_t gemm_pair(const uint16_t* A, const uint16_t* A2, const uint16_t* B, int64_t R, int64_t SN, int64_t T,
                     float* C, const float* alpha_dev, float alpha_host, hipStream_t s) {
    if (((R + 255) / 256) * ((SN + 255) / 256) >= 256)
        return gemm_pair_shape<4, 4, 2>(A, A2, B, R, SN, T, C, alpha_dev, alpha_host, s);
    return gemm_pair_shape<2, 2, 2>(A, A2, B, R, SN, T, C, alpha_dev, alpha_host, s);
}

// ------------------------------------------------------ rows: H and norm ----
// One workgroup per row: dZ (fp32, read from and replaced in dzx) -> dR = H dZ
// with the forward's register / LDS butterflies (act_row.h), then the norm's
// backward with the row's x and gain at the same element positions.
template <int LK, int NT, typename Tx, bool HAD>
__global__ __launch_bounds__(NT) void bwd_rows_kernel(float* __restrict__ dzx, const Tx* __restrict__ X,
                                                      const float* __restrict__ gain, int norm, float norm_eps) {
    using S = ActShape<LK, NT, float>;
    constexpr int K = S::K, E = S::E, V = S::V, LV = S::LV, LT = S::LT, VB = S::VB, VW = S::VW, FREE = S::FREE;
    constexpr int NVEC = E / VW;
    using Ph = Phases<NT, E, VB, FREE, LV, LV + LT>;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ double red[NT / kWave];
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    float* drow = dzx + row * K;
    const Tx* xrow = X + row * K;
    ActRegs<LK, NT, float> v;
    act_row_load<LK, NT, float>(drow, v);
    if constexpr (HAD) {
        reg_fwht<E>(v);
        float* const base = lds + lds_off<VW>(tid * V);  // the thread's part of the offsets (see phase_elem)
#pragma unroll
        for (int c = 0; c < S::C; c++)
#pragma unroll
            for (int j = 0; j < V; j += VW) {
                float* p = base + lds_off<VW>(c * NT * V + j);
                *reinterpret_cast<float4*>(p) = make_float4(v[c * V + j], v[c * V + j + 1], v[c * V + j + 2], v[c * V + j + 3]);
            }
        __syncthreads();
        Ph::run(lds, v);
        const float inv = 1.f / sqrtf((float)K);
#pragma unroll
        for (int e = 0; e < E; e++) v[e] *= inv;
    }
    constexpr int SLO = HAD ? Ph::LAST_LO : 0;
    constexpr int SR = HAD ? Ph::LAST_R : 0;
    auto pos = [&](int u) {  // element index of register vector u
        if constexpr (HAD) {
            return phase_base<NT, VB, SLO, SR>(u >> SR, u & ((1 << SR) - 1));
        } else {
            const int j = u * VW;
            return ((j / V) * NT + tid) * V + (j % V);
        }
    };
    // x at the same positions; v becomes a = g * dR (every formula below uses
    // the gain only in that product), then the output, in place
    float x[E];
#pragma unroll
    for (int u = 0; u < NVEC; u++) {
        const int e0 = pos(u);
        if constexpr (sizeof(Tx) == 4) {
            const float4 q = *reinterpret_cast<const float4*>(xrow + e0);
            x[4 * u] = q.x; x[4 * u + 1] = q.y; x[4 * u + 2] = q.z; x[4 * u + 3] = q.w;
        } else {
            const uint2 q = *reinterpret_cast<const uint2*>(xrow + e0);
            x[4 * u] = bf16_lo(q.x); x[4 * u + 1] = bf16_hi(q.x); x[4 * u + 2] = bf16_lo(q.y); x[4 * u + 3] = bf16_hi(q.y);
        }
        if (gain) {
#pragma unroll
            for (int t = 0; t < 4; t++) v[4 * u + t] *= gain[e0 + t];
        }
    }
    // per-thread sums in fp32 (at most 64 terms), the block's sums in fp64
    if (norm == HBL_NORM_RMS) {
        float ss = 0.f, t = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) {
            ss += x[e] * x[e];
            t += v[e] * x[e];
        }
        const double sst = block_sum_f64<NT>((double)ss, red);
        const double tt = block_sum_f64<NT>((double)t, red);
        const double c = 1.0 / sqrt(sst / K + (double)norm_eps);
        const float cf = (float)c, kf = (float)(c * c * c / K * tt);
#pragma unroll
        for (int e = 0; e < E; e++) v[e] = cf * v[e] - kf * x[e];
    } else if (norm == HBL_NORM_LN) {
        float s1 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) s1 += x[e];
        const float mu = (float)(block_sum_f64<NT>((double)s1, red) / K);
        float s2 = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) {
            x[e] -= mu;
            s2 += x[e] * x[e];
        }
        const float c = (float)(1.0 / sqrt(block_sum_f64<NT>((double)s2, red) / K + (double)norm_eps));
        float sa = 0.f, sax = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) {
            x[e] *= c;  // xh
            sa += v[e];
            sax += v[e] * x[e];
        }
        const float ma = (float)(block_sum_f64<NT>((double)sa, red) / K);
        const float mx = (float)(block_sum_f64<NT>((double)sax, red) / K);
#pragma unroll
        for (int e = 0; e < E; e++) v[e] = c * (v[e] - ma - x[e] * mx);
    }
    __syncthreads();  // every thread has read its dZ values (the row is rewritten in place)
#pragma unroll
    for (int u = 0; u < NVEC; u++)
        *reinterpret_cast<float4*>(drow + pos(u)) = make_float4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
}

template <int LK, typename Tx, bool HAD>
hipError_t launch_rows(float* dzx, int64_t M, const Tx* X, const float* gain, const hbl_config& cfg, hipStream_t s) {
    constexpr int NT = threads_for(LK);
    static_assert(ActShape<LK, NT, float>::VW == 4, "four values per vector");
    const size_t lds_bytes = HAD ? (size_t)ActShape<LK, NT, float>::lds_floats * sizeof(float) : 0;
    auto kern = bwd_rows_kernel<LK, NT, Tx, HAD>;
    static std::atomic<uint32_t> lds_set{0};  // devices with the LDS limit raised for this kernel
    if (hipError_t e = set_dynamic_lds(kern, lds_bytes, lds_set); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)M), dim3(NT), lds_bytes, s, dzx, X, gain, cfg.norm, cfg.norm_eps);
    return hipGetLastError();
}

template <typename Tx, bool HAD>
hipError_t rows_k(float* dzx, int64_t M, int64_t K, const Tx* X, const float* gain, const hbl_config& cfg,
                  hipStream_t s) {
    switch (K) {
        case 512: return launch_rows<9, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 1024: return launch_rows<10, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 2048: return launch_rows<11, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 4096: return launch_rows<12, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 8192: return launch_rows<13, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 16384: return launch_rows<14, Tx, HAD>(dzx, M, X, gain, cfg, s);
        case 32768: return launch_rows<15, Tx, HAD>(dzx, M, X, gain, cfg, s);
        default: return hipErrorInvalidValue;
    }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

int64_t bwd_pad64(int64_t v) { return (v + 63) / 64 * 64; }  // whole GEMM K steps

size_t backward_ws_bytes(int64_t M, int64_t K, int64_t N, int act_bits, bool want_dw) {
    auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
    const int64_t Np = bwd_pad64(N), Mp = bwd_pad64(M);
    size_t b = r256((size_t)K * Np * 2) + 2 * r256((size_t)M * Np * 2);
    if (want_dw)
        b += r256((size_t)M * K * act_bits / 8) + r256((size_t)M * 4) + r256((size_t)K * Mp * 2) +
             2 * r256((size_t)Np * Mp * 2);
    return b;
}

hipError_t launch_backward(const void* dY, int dy_dtype, const void* X, int x_dtype, int64_t M, int64_t K,
                           const float* gain, const uint8_t* W_packed, const float* alpha, int64_t N,
                           const hbl_config& cfg, float* dX, float* dW, void* ws, hipStream_t s) {
    auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
    const int64_t Np = bwd_pad64(N), Mp = bwd_pad64(M);
    uint8_t* p = (uint8_t*)ws;
    uint16_t* Wt = (uint16_t*)p; p += r256((size_t)K * Np * 2);
    uint16_t* Yh = (uint16_t*)p; p += r256((size_t)M * Np * 2);
    uint16_t* Yl = (uint16_t*)p; p += r256((size_t)M * Np * 2);
    const bool split = dy_dtype == HBL_F32;  // a bf16 dY is exact in one bf16 operand
    hipError_t e = hipSuccess;
    // weights: 2-bit [N][K/4] -> bf16 [K][Np]
    convert_transpose(TernSrc{(const uint32_t*)W_packed, K}, N, K, Wt, nullptr, Np, s);
    // dY -> bf16 [M][Np] (+ remainder)
    if (dy_dtype == HBL_F32)
        hipLaunchKernelGGL(split_bf16_kernel<float>, dim3((unsigned)M, blocks_for(Np / 8)), dim3(256), 0, s, (const float*)dY, M, N,
                           Np, (const float*)nullptr, Yh, Yl);
    else
        hipLaunchKernelGGL(split_bf16_kernel<uint16_t>, dim3((unsigned)M, blocks_for(Np / 8)), dim3(256), 0, s,
                           (const uint16_t*)dY, M, N, Np, (const float*)nullptr, Yh, (uint16_t*)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // dZ = alpha * dY . Wq  -> dX (fp32 [M][K]), then H and the norm in place
    if ((e = gemm_pair(Yh, split ? Yl : nullptr, Wt, M, K, Np, dX, alpha, 0.f, s)) != hipSuccess) return e;
    if (x_dtype == HBL_F32)
        e = cfg.hadamard ? rows_k<float, true>(dX, M, K, (const float*)X, gain, cfg, s)
                         : rows_k<float, false>(dX, M, K, (const float*)X, gain, cfg, s);
    else
        e = cfg.hadamard ? rows_k<uint16_t, true>(dX, M, K, (const uint16_t*)X, gain, cfg, s)
                         : rows_k<uint16_t, false>(dX, M, K, (const uint16_t*)X, gain, cfg, s);
    if (e != hipSuccess || !dW) return e;
    // dW = (dY * d)^T . q: the forward's codes and scales again
    uint8_t* codes = p; p += r256((size_t)M * K * cfg.act_bits / 8);
    float* xs = (float*)p; p += r256((size_t)M * 4);
    uint16_t* Qt = (uint16_t*)p; p += r256((size_t)K * Mp * 2);
    uint16_t* PTh = (uint16_t*)p; p += r256((size_t)Np * Mp * 2);
    uint16_t* PTl = (uint16_t*)p;
    if ((e = launch_act_quant(X, x_dtype, M, K, gain, cfg, codes, xs, nullptr, nullptr, s)) != hipSuccess) return e;
    // codes -> bf16 [K][Mp]; P = dY * d as bf16 high part + remainder, [Np][Mp]
    if (cfg.act_bits == 8) convert_transpose(CodesSrc<8>{codes, K}, M, K, Qt, nullptr, Mp, s);
    else convert_transpose(CodesSrc<4>{codes, K}, M, K, Qt, nullptr, Mp, s);
    if (dy_dtype == HBL_F32) convert_transpose(SplitSrc<float>{(const float*)dY, N, xs}, M, N, PTh, PTl, Mp, s);
    else convert_transpose(SplitSrc<uint16_t>{(const uint16_t*)dY, N, xs}, M, N, PTh, PTl, Mp, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return gemm_pair(PTh, PTl, Qt, N, K, Mp, dW, nullptr, 1.f, s);
}

}  // namespace hbl
