// int_dot.h -- integer operand unpacking, rescale and the small-M GEMV
// routines shared by the GEMM kernels and the fused small-M forward (gfx950).
// Internal header.
//
// Operand unpack (in registers):
//   * weights: one 32-bit word holds an aligned group of 16 trits, byte b
//     holding k = b, b+4, b+8, b+12 in its bit pairs.  (word << (6-2c)) &
//     0xC0C0C0C0 puts the trits k = 4c..4c+3 in the top two bits of bytes
//     0..3: as int8 that is 64 * w.  Four such dwords are 16 int8 operands
//     in natural k order.
//   * INT8 codes are used as loaded (natural k order).
//   * INT4 codes (low nibble = even k) are spread with v_perm so that each
//     code lands in the top nibble of its byte: as int8 that is 16 * q.
// Integer products therefore accumulate 64*acc (INT8) or 1024*acc (INT4),
// exact in int32 for K <= 32768, and the epilogue shifts them back.  The
// rescale is y = fp32(fp32(acc * xscale[m]) * alpha) (no bias: the
// "新智元: 微软 BitNet v2" repost, section "BitNet v2：原生4位激活").
#pragma once
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

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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

// ============================================================ small-M GEMV ==
// M <= 4 tokens, K a power of two in [1024, 16384]: a matrix-vector product
// on the vector ALU (v_dot4_i32_i8), so that the weight stream is read with
// fully coalesced 16-byte loads like a plain copy.  One block of T threads
// per 16 output columns; the block's 16 weight rows are contiguous in memory
// (16 * K/4 bytes).  Vector v of that slice (64 trits) is row v / CPR, chunk
// v % CPR, with CPR = K/64 chunks per row; thread t takes v = t + T j, so
// it always sees chunk c = t % CPR (one set of activation codes, kept in
// registers) of rows t / CPR + j * (T / CPR).  Each instruction of a wave
// reads 1 KiB of consecutive bytes.  Partial dot products are summed over the
// CPR threads of a row: DPP adds inside each 16-lane row, then LDS.
constexpr int kGvRows = 16, kGvMaxM = 4;

// Sum over the 16 lanes of a DPP row (every lane of the row gets the sum):
// swap neighbours, swap pairs, rotate the row by 4, rotate it by 8.
HBL_DEVINL int row16_sum(int x) {
    x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_mov_dpp(x, 0x124, 0xF, 0xF, false);  // row_ror:4
    x += __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
    return x;
}

// The GEMV of one block: T threads, 16 weight rows, up to MS tokens, K = 64 << LCPR.
template <int BITS, int LCPR, int MS, int T>
struct Gv {
    static constexpr int CPR = 1 << LCPR;          // 64-trit chunks per weight row
    static constexpr int K = 64 * CPR;
    static constexpr int V = kGvRows * CPR / T;    // weight vectors per thread
    static constexpr int RS = T / CPR;             // row stride between a thread's vectors
    static constexpr int ABytes = 64 * BITS / 8;   // code bytes per chunk and token
    static constexpr int AVecs = ABytes / 16;
    static_assert(V >= 1 && RS >= 1 && RS * V == kGvRows, "unsupported K for this thread count");
    using WRegs = uint4[V];
    using ARegs = uint4[MS][AVecs];
    using AOps = v4i[MS][4];
    using Acc = int[V][MS];
    using Part = int[V][MS][T / 16];

    static HBL_DEVINL int chunk() { return (int)threadIdx.x & (CPR - 1); }

    // codes of this thread's chunk for each token, from global memory (tokens past M: zeros)
    static HBL_DEVINL void load_codes(const uint8_t* __restrict__ A, int M, ARegs& a) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(A, (int64_t)M * (K * BITS / 8));
#pragma unroll
        for (int m = 0; m < MS; m++)
#pragma unroll
            for (int q = 0; q < AVecs; q++)
                a[m][q] = buf_load16(rs, (uint32_t)(m * (K * BITS / 8) + chunk() * ABytes + q * 16));
    }
    // the same from a [MS][K*BITS/8] block of LDS whose first M rows are valid
    static HBL_DEVINL void load_codes_lds(const uint8_t* codes, int M, ARegs& a) {
#pragma unroll
        for (int m = 0; m < MS; m++)
#pragma unroll
            for (int q = 0; q < AVecs; q++)
                a[m][q] = m < M ? *reinterpret_cast<const uint4*>(codes + m * (K * BITS / 8) + chunk() * ABytes + q * 16)
                                : make_uint4(0, 0, 0, 0);
    }
    // the block's 16 weight rows (contiguous, 16 * K/4 bytes from row n0)
    static HBL_DEVINL void load_w(const uint8_t* __restrict__ Wp, int64_t n0, WRegs& w) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(Wp + n0 * (K / 4), (int64_t)kGvRows * (K / 4));
#pragma unroll
        for (int j = 0; j < V; j++) w[j] = buf_load16(rs, (uint32_t)(((int)threadIdx.x + j * T) * 16));
    }
    // activation operands of the chunk's four 16-k groups, as int8 dwords
    static HBL_DEVINL void unpack_codes(const ARegs& a, AOps& av) {
#pragma unroll
        for (int m = 0; m < MS; m++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if constexpr (BITS == 8) {
                    const uint4 q = a[m][i];
                    av[m][i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
                } else {
                    const uint4 q = a[m][i / 2];
                    av[m][i] = (i & 1) ? unpack_a4(q.z, q.w) : unpack_a4(q.x, q.y);
                }
            }
    }
    // dot products, weight vectors in issue order
    static HBL_DEVINL void dot(const WRegs& w, const AOps& av, Acc& acc) {
#pragma unroll
        for (int j = 0; j < V; j++) {
#pragma unroll
            for (int m = 0; m < MS; m++) acc[j][m] = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {  // 16-k group i of the chunk
                const uint32_t word = i == 0 ? w[j].x : i == 1 ? w[j].y : i == 2 ? w[j].z : w[j].w;
                const v4i b = unpack_w(word);
#pragma unroll
                for (int m = 0; m < MS; m++) {
                    int t = acc[j][m];
#pragma unroll
                    for (int d = 0; d < 4; d++) t = __builtin_amdgcn_sdot4(b[d], av[m][i][d], t, false);
                    acc[j][m] = t;
                }
            }
        }
    }
    // Sum over the CPR threads of a row group (DPP adds over each 16-lane row,
    // then the row sums through LDS; exact integer adds), rescale, store Y
    // rows n0..n0+15 of the first M tokens.  xs may point to global or LDS.
    template <typename YT>
    static HBL_DEVINL void finish(Acc& acc, Part& part, int M, const float* xs, float alpha, int64_t N,
                                  YT* __restrict__ Y, int64_t n0) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < V; j++)
#pragma unroll
            for (int m = 0; m < MS; m++) {
                const int t = row16_sum(acc[j][m]);
                if ((tid & 15) == 0) part[j][m][tid >> 4] = t;
            }
        __syncthreads();
        // output (row r, token m): row group r % RS owns the 16-lane rows
        // (r % RS) * CPR/16 .. +CPR/16-1; vector j = r / RS
        if (tid < kGvRows * MS) {
            const int r = tid / MS, m = tid % MS;
            const int gr = r % RS, j = r / RS;
            int sum = 0;
#pragma unroll
            for (int x = 0; x < CPR / 16; x++) sum += part[j][m][gr * (CPR / 16) + x];
            if (m < M) store_y<YT>(Y + m * N + n0 + r, rescale(sum >> Shift<BITS>::value, xs[m], alpha));
        }
    }
};

}  // namespace
}  // namespace hbl
