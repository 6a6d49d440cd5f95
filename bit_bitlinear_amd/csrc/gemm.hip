// gemm.hip -- INT8/INT4 activation codes x ternary 2-bit weights on the gfx950
// i8 matrix cores, int32 accumulation, fused rescale epilogue.
//
// The "新智元: 微软 BitNet v2" repost (section "原生4比特盘算") argues that dense
// low-bit compute, not sparsity, serves batched inference; the product
// acc[m][n] = sum_k q[m][k] W_q[n][k] is therefore a dense integer contraction
// and runs on MFMA.  The epilogue applies y = fp32(fp32(acc * xscale[m]) * alpha)
// (no bias: section "BitNet v2：原生4位激活").
//
// Operand unpack (in registers, per wave):
//   * weights: one 32-bit word holds an aligned group of 16 trits, byte b
//     holding k = b, b+4, b+8, b+12 in its bit pairs.  (word << (6-2c)) &
//     0xC0C0C0C0 puts the trits k = 4c..4c+3 in the top two bits of bytes
//     0..3: as int8 that is 64 * w.  Four such dwords form one 16-byte MFMA
//     operand in natural k order.
//   * INT8 codes are used as loaded (natural k order).
//   * INT4 codes (low nibble = even k) are spread with v_perm so that each
//     code lands in the top nibble of its byte: as int8 that is 16 * q.
// The i8 MFMA therefore accumulates 64*acc (INT8) or 1024*acc (INT4), exact
// in int32 for K <= 32768, and the epilogue shifts it back.
// For a given lane both operands hold the same k set, so the k order inside
// an operand does not matter to the result.
#include "hbl_device.h"

namespace hbl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

HBL_DEVINL v4i unpack_w(uint32_t y) {
    v4i r;
    r[0] = (int)((y << 6) & 0xC0C0C0C0u);
    r[1] = (int)((y << 4) & 0xC0C0C0C0u);
    r[2] = (int)((y << 2) & 0xC0C0C0C0u);
    r[3] = (int)(y & 0xC0C0C0C0u);
    return r;
}

// 16 INT4 codes (k ascending, low nibble first) -> 16 bytes, code in the top nibble.
HBL_DEVINL v4i unpack_a4(uint32_t x0, uint32_t x1) {
    const uint32_t l0 = x0 << 4, l1 = x1 << 4;
    v4i r;
    r[0] = (int)(__builtin_amdgcn_perm(x0, l0, 0x05010400u) & 0xF0F0F0F0u);
    r[1] = (int)(__builtin_amdgcn_perm(x0, l0, 0x07030602u) & 0xF0F0F0F0u);
    r[2] = (int)(__builtin_amdgcn_perm(x1, l1, 0x05010400u) & 0xF0F0F0F0u);
    r[3] = (int)(__builtin_amdgcn_perm(x1, l1, 0x07030602u) & 0xF0F0F0F0u);
    return r;
}

template <int BITS>
struct Shift {
    static constexpr int value = BITS == 8 ? 6 : 10;
};

template <typename YT>
HBL_DEVINL void store_y(YT* p, float v);
template <>
HBL_DEVINL void store_y<float>(float* p, float v) { *p = v; }
template <>
HBL_DEVINL void store_y<uint16_t>(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }

HBL_DEVINL float rescale(int acc, float d, float alpha) {
    const float t = (float)acc * d;  // two separately rounded fp32 products
    return t * alpha;
}

// ============================================================ prefill GEMM ==
// Block tile 128 x 128, K step 64, 4 waves in a 2 x 2 grid, each wave 64 x 64
// = 2 x 2 MFMA 32x32x32 tiles.  Packed A and W tiles are staged in LDS (double
// buffered) and unpacked in registers right before the MFMA.
constexpr int kBM = 128, kBN = 128, kBK = 64, kGemmThreads = 256;

template <int BITS>
struct ATile {
    static constexpr int row_bytes = BITS == 8 ? kBK : kBK / 2;  // bytes of one row per K step
    static constexpr int stride = row_bytes + 16;                // padded LDS row
    static constexpr int chunks = kBM * row_bytes / 16;          // 16-byte chunks per tile
};
constexpr int kBStride = 20;  // 16 bytes of packed W per row and K step, padded to 5 dwords

template <int BITS, typename YT>
__global__ __launch_bounds__(kGemmThreads) void gemm_mfma_kernel(const uint8_t* __restrict__ A,
                                                                 const float* __restrict__ xscale, int64_t M,
                                                                 int64_t K, const uint8_t* __restrict__ Wp,
                                                                 const float* __restrict__ alpha_p, int64_t N,
                                                                 YT* __restrict__ Y) {
    using AT = ATile<BITS>;
    __shared__ __attribute__((aligned(16))) uint8_t As[2][kBM * AT::stride];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][kBN * kBStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t a_ld = K * BITS / 8;  // bytes per activation row
    const int64_t w_ld = K / 4;         // bytes per weight row
    const int KT = (int)(K / kBK);

    constexpr int A_PER_THREAD = (AT::chunks + kGemmThreads - 1) / kGemmThreads;
    constexpr int A_CPR = AT::row_bytes / 16;  // chunks per row
    uint4 a_reg[A_PER_THREAD];
    uint4 b_reg;

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int r = 0; r < A_PER_THREAD; r++) {
            const int q = tid + r * kGemmThreads;
            const int row = q / A_CPR, c16 = q % A_CPR;
            const int64_t m = m0 + row;
            a_reg[r] = m < M ? *reinterpret_cast<const uint4*>(A + m * a_ld + (int64_t)kt * AT::row_bytes + c16 * 16)
                             : make_uint4(0, 0, 0, 0);
        }
        if (tid < kBN) {
            const int64_t n = n0 + tid;
            b_reg = n < N ? *reinterpret_cast<const uint4*>(Wp + n * w_ld + (int64_t)kt * (kBK / 4))
                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int st) {
#pragma unroll
        for (int r = 0; r < A_PER_THREAD; r++) {
            const int q = tid + r * kGemmThreads;
            const int row = q / A_CPR, c16 = q % A_CPR;
            *reinterpret_cast<uint4*>(&As[st][row * AT::stride + c16 * 16]) = a_reg[r];
        }
        if (tid < kBN) {
            uint32_t* d = reinterpret_cast<uint32_t*>(&Bs[st][tid * kBStride]);
            d[0] = b_reg.x; d[1] = b_reg.y; d[2] = b_reg.z; d[3] = b_reg.w;
        }
    };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int lr = lane & 31;  // row (A) / column (W) inside a 32-wide MFMA tile
    const int lg = lane >> 5;  // which 16-k half of the 32-k MFMA step
    for (int kt = 0; kt < KT; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
        for (int s = 0; s < kBK / 32; s++) {
            v4i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int row = wm * 64 + i * 32 + lr;
                if constexpr (BITS == 8) {
                    const uint4 q = *reinterpret_cast<const uint4*>(&As[cur][row * AT::stride + s * 32 + lg * 16]);
                    a[i][0] = (int)q.x; a[i][1] = (int)q.y; a[i][2] = (int)q.z; a[i][3] = (int)q.w;
                } else {
                    const uint2 q = *reinterpret_cast<const uint2*>(&As[cur][row * AT::stride + s * 16 + lg * 8]);
                    a[i] = unpack_a4(q.x, q.y);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int col = wn * 64 + j * 32 + lr;
                const uint32_t y = *reinterpret_cast<const uint32_t*>(&Bs[cur][col * kBStride + s * 8 + lg * 4]);
                b[j] = unpack_w(y);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds column lr, rows 8*(r/4) + 4*lg + r%4 of each 32x32 tile
    const float alpha = *alpha_p;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t n = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
                if (m < M && n < N) {
                    const int v = acc[i][j][r] >> Shift<BITS>::value;
                    store_y<YT>(Y + m * N + n, rescale(v, xscale[m], alpha));
                }
            }
        }
    }
}

// ============================================================ decode GEMM ==
// M <= 64 tokens.  The weights dominate the traffic, so the kernel streams W
// once: one block per 16 output columns, its 4 waves split K (wave w takes the
// 64-wide K steps w, w+4, ...), each K step is one MFMA 16x16x64 per 16-row
// token tile.  The partial accumulators of the 4 waves are summed in LDS
// (int32, exact) before the rescale.
constexpr int kDecThreads = 256, kDecBN = 16, kDecUnroll = 4;

template <int BITS, int MT, typename YT>
__global__ __launch_bounds__(kDecThreads) void gemm_decode_kernel(const uint8_t* __restrict__ A,
                                                                  const float* __restrict__ xscale, int64_t M,
                                                                  int64_t K, const uint8_t* __restrict__ Wp,
                                                                  const float* __restrict__ alpha_p, int64_t N,
                                                                  YT* __restrict__ Y) {
    __shared__ int red[4][MT][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;  // token row (A) / weight column (W) inside the tile
    const int lg = lane >> 4;   // which 16-k quarter of the 64-k step
    const int64_t n = (int64_t)blockIdx.x * kDecBN + l16;
    const int64_t a_ld = K * BITS / 8;
    const int64_t w_ld = K / 4;
    const int KS = (int)(K / 64);

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) acc[t] = v4i{0, 0, 0, 0};

    const uint8_t* wrow = Wp + n * w_ld + lg * 4;  // 16 trits = 4 bytes per lane per K step
    int ks = wave;
    for (; ks + 4 * (kDecUnroll - 1) < KS; ks += 4 * kDecUnroll) {
        uint32_t wv[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; u++) wv[u] = *reinterpret_cast<const uint32_t*>(wrow + (ks + 4 * u) * 16);
#pragma unroll
        for (int u = 0; u < kDecUnroll; u++) {
            const v4i b = unpack_w(wv[u]);
            const int64_t k0 = (int64_t)(ks + 4 * u) * 64 + lg * 16;
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const int64_t m = t * 16 + l16;
                v4i a = v4i{0, 0, 0, 0};
                if (m < M) {
                    if constexpr (BITS == 8) {
                        const uint4 q = *reinterpret_cast<const uint4*>(A + m * a_ld + k0);
                        a[0] = (int)q.x; a[1] = (int)q.y; a[2] = (int)q.z; a[3] = (int)q.w;
                    } else {
                        const uint2 q = *reinterpret_cast<const uint2*>(A + m * a_ld + k0 / 2);
                        a = unpack_a4(q.x, q.y);
                    }
                }
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
            }
        }
    }
    for (; ks < KS; ks += 4) {
        const v4i b = unpack_w(*reinterpret_cast<const uint32_t*>(wrow + ks * 16));
        const int64_t k0 = (int64_t)ks * 64 + lg * 16;
#pragma unroll
        for (int t = 0; t < MT; t++) {
            const int64_t m = t * 16 + l16;
            v4i a = v4i{0, 0, 0, 0};
            if (m < M) {
                if constexpr (BITS == 8) {
                    const uint4 q = *reinterpret_cast<const uint4*>(A + m * a_ld + k0);
                    a[0] = (int)q.x; a[1] = (int)q.y; a[2] = (int)q.z; a[3] = (int)q.w;
                } else {
                    const uint2 q = *reinterpret_cast<const uint2*>(A + m * a_ld + k0 / 2);
                    a = unpack_a4(q.x, q.y);
                }
            }
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
        }
    }

#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int r = 0; r < 4; r++) red[wave][t][r][lane] = acc[t][r];
    __syncthreads();
    // wave w finishes token tiles t = w, w+4, ... (output: column l16, rows 4*lg + r)
    const float alpha = *alpha_p;
    for (int t = wave; t < MT; t += 4) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int sum = red[0][t][r][lane] + red[1][t][r][lane] + red[2][t][r][lane] + red[3][t][r][lane];
            const int64_t m = t * 16 + 4 * lg + r;
            if (m < M && n < N) store_y<YT>(Y + m * N + n, rescale(sum >> Shift<BITS>::value, xscale[m], alpha));
        }
    }
}

template <int BITS, typename YT>
hipError_t launch_typed(const uint8_t* A, const float* xscale, int64_t M, int64_t K, const uint8_t* Wp,
                        const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    if (M <= 64) {
        const dim3 grid((unsigned)((N + kDecBN - 1) / kDecBN));
        if (M <= 16)
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, 1, YT>), grid, dim3(kDecThreads), 0, s, A, xscale, M, K, Wp,
                               alpha, N, Y);
        else if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, 2, YT>), grid, dim3(kDecThreads), 0, s, A, xscale, M, K, Wp,
                               alpha, N, Y);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, 4, YT>), grid, dim3(kDecThreads), 0, s, A, xscale, M, K, Wp,
                               alpha, N, Y);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
    hipLaunchKernelGGL((gemm_mfma_kernel<BITS, YT>), grid, dim3(kGemmThreads), 0, s, A, xscale, M, K, Wp, alpha, N,
                       Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* codes, const float* xscale, int act_bits, int64_t M, int64_t K,
                       const uint8_t* W_packed, const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const uint8_t* A = (const uint8_t*)codes;
    if (act_bits == 8) {
        return y_dtype == HBL_F32 ? launch_typed<8, float>(A, xscale, M, K, W_packed, alpha, N, (float*)Y, s)
                                  : launch_typed<8, uint16_t>(A, xscale, M, K, W_packed, alpha, N, (uint16_t*)Y, s);
    }
    return y_dtype == HBL_F32 ? launch_typed<4, float>(A, xscale, M, K, W_packed, alpha, N, (float*)Y, s)
                              : launch_typed<4, uint16_t>(A, xscale, M, K, W_packed, alpha, N, (uint16_t*)Y, s);
}

}  // namespace hbl
