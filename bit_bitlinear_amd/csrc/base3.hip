// base3.hip -- ternary weights stored five per byte, and the small-M GEMV
// that reads them (gfx950).
//
// Storage (the CSDN post "[论文品鉴] 1-bit LLM", section "掩码存储": several
// ternary weights packed into one integer, five per 8-bit byte): byte j of a
// row holds the weights k = 5j .. 5j+4 as base-3 digits t + 1, the first
// weight least significant, byte = sum_i (t_i + 1) 3^i; weights past K are 0
// (digit 1) and every row is padded to whole 16-byte vectors of 80 weights
// (16 * ceil(K/80) bytes, 1.6 bits per weight against 2 for the 2-bit format).
//
// GEMV (M <= 4 tokens, K <= 16384): one lane per 16-byte vector position p of
// a row (T = 64, 128 or 256 threads, the least that covers the row), R rows
// per block.  A lane loads
// the codes of its 80 positions once (from L2) and the R weight vectors of
// its position up front, so every wave instruction reads 1 KiB of
// consecutive weight bytes.  A byte becomes its five int8 weights by one
// 8-byte LDS table read; the four tables (one per byte position j in a
// 32-bit word) place the five weights at bytes j .. j+4 of the entry, so the
// 20 weights of a word are five dwords formed by three ORs:
//   d0 = E0.lo, d1 = E0.hi | E1.lo, d2 = E1.hi | E2.lo, d3 = E2.hi | E3.lo, d4 = E3.hi.
// Products run on v_dot4_i32_i8 with exact int32 sums, summed over the lanes
// of a row (DPP inside 16-lane rows, then LDS) and rescaled exactly as the
// other GEMM paths do, so the output equals theirs bit for bit.
#include <hip/hip_runtime.h>

#include "hbl.h"
#include "hbl_device.h"
#include "int_dot.h"

namespace hbl {
namespace {

typedef unsigned int v2u_b3 __attribute__((ext_vector_type(2)));

HBL_DEVINL uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v2u_b3 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v[0], v[1]);
}

// ------------------------------------------------------------ packing ----
// One thread per output vector (row n, position p): the 80 weights
// k = 80p .. 80p+79 are the five 16-groups 5p .. 5p+4 of the 2-bit row
// (in each group, weight e at bits 8*(e%4) + 2*(e/4); 00 -> 0, 01 -> +1,
// 11 -> -1; groups past K read as zeros, i.e. weight 0).
__global__ __launch_bounds__(256) void pack_base3_kernel(const uint32_t* __restrict__ Wp, int64_t N, int64_t K,
                                                         int vpr, uint4* __restrict__ W3) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * vpr) return;
    const int64_t n = i / vpr;
    const int p = (int)(i - n * vpr);
    const int64_t gpr = K / 16;
    uint32_t wd[5];
#pragma unroll
    for (int g = 0; g < 5; g++) {
        const int64_t gi = (int64_t)p * 5 + g;
        wd[g] = gi < gpr ? Wp[n * gpr + gi] : 0u;
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; j++) {
        uint32_t byte = 0, place = 1;
#pragma unroll
        for (int d = 0; d < 5; d++) {
            const int k = 5 * j + d, e = k & 15;
            const uint32_t c = (wd[k >> 4] >> (8 * (e & 3) + 2 * (e >> 2))) & 3u;
            byte += ((c + 1u) & 3u) * place;  // 00 -> 1, 01 -> 2, 11 -> 0: the digit t + 1
            place *= 3u;
        }
        out[j >> 2] |= byte << (8 * (j & 3));
    }
    W3[i] = make_uint4(out[0], out[1], out[2], out[3]);
}

// --------------------------------------------------------------- GEMV ----
constexpr int kB3Rows = 4;  // weight rows per block (8: +20% time at 1 x 8192 x 4096, fewer waves per CU)

// Byte -> its five weights as int8 at bytes j .. j+4 of table j's 8-byte
// entry (j = 0..3, the byte's position in a 32-bit word); bytes above 242
// never occur and map to 0.  Built at compile time; each block copies the
// 8 KiB into LDS.
struct B3Lut {
    uint32_t w[4][256][2];
};
constexpr B3Lut make_b3_lut() {
    B3Lut t{};
    for (int j = 0; j < 4; j++)
        for (int b = 0; b < 256; b++) {
            uint64_t v = 0;
            if (b < 243) {
                int x = b;
                for (int i = 0; i < 5; i++) {
                    const int tr = x % 3 - 1;
                    x /= 3;
                    v |= (uint64_t)(uint8_t)(int8_t)tr << (8 * (j + i));
                }
            }
            t.w[j][b][0] = (uint32_t)v;
            t.w[j][b][1] = (uint32_t)(v >> 32);
        }
    return t;
}
__device__ const B3Lut kB3Lut = make_b3_lut();

template <int BITS, int MS, int T, int R, typename YT>
__global__ __launch_bounds__(T) void gemv_base3_kernel(const uint8_t* __restrict__ A, const float* __restrict__ xs,
                                                       int M, int K, int vpr, const uint8_t* __restrict__ W3,
                                                       const float* __restrict__ alpha_p, int64_t N,
                                                       YT* __restrict__ Y) {
    __shared__ uint2 lut[4][256];
    __shared__ int part[R][MS][T / 16];
    const int tid = threadIdx.x;
    const bool live = tid < vpr;  // lane tid owns vector position tid of every row
    const int64_t n0 = (int64_t)blockIdx.x * R;
    const int64_t rb = 16 * (int64_t)vpr;
    const int64_t a_ld = (int64_t)K * BITS / 8;

    // the decode tables first (8 KiB, from L2 after the first blocks), so
    // that storing them to LDS waits only for these loads
    constexpr int kLv = (int)(sizeof(B3Lut) / 16), LI = kLv / T;
    static_assert(kLv % T == 0, "whole table vectors per thread");
    const uint4* tg = reinterpret_cast<const uint4*>(&kB3Lut) + tid;
    uint4 tl[LI];
#pragma unroll
    for (int i = 0; i < LI; i++) tl[i] = tg[i * T];
    // the codes of positions 80 tid .. +79 for each token (tokens >= M and
    // bytes past the buffer read as zeros; codes past K meet zero weights)
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)M * a_ld);
    uint32_t a[MS][20];
    uint2 a4raw[BITS == 4 ? MS : 1][5];
#pragma unroll
    for (int m = 0; m < MS; m++) {
        if constexpr (BITS == 8) {
#pragma unroll
            for (int v = 0; v < 5; v++) {
                const uint4 q = buf_load16(ra, (uint32_t)(m * a_ld + 80 * tid + 16 * v));
                a[m][4 * v] = q.x; a[m][4 * v + 1] = q.y; a[m][4 * v + 2] = q.z; a[m][4 * v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < 5; v++) a4raw[m][v] = buf_load8(ra, (uint32_t)(m * a_ld + 40 * tid + 8 * v));
        }
    }
    // the block's weight rows at this lane's position (rows past N read as zeros)
    const int64_t rows = N - n0 < R ? N - n0 : R;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W3 + n0 * rb, rows * rb);
    uint4 w[R];
#pragma unroll
    for (int r = 0; r < R; r++) w[r] = buf_load16(rw, (uint32_t)(r * rb + 16 * tid));

#pragma unroll
    for (int i = 0; i < LI; i++) reinterpret_cast<uint4*>(&lut[0][0])[tid + i * T] = tl[i];
    __syncthreads();

    if constexpr (BITS == 4) {
#pragma unroll
        for (int m = 0; m < MS; m++)
#pragma unroll
            for (int v = 0; v < 5; v++) {
                const v4i u = unpack_a4(a4raw[m][v].x, a4raw[m][v].y);  // 16 * q
                a[m][4 * v] = (uint32_t)u[0]; a[m][4 * v + 1] = (uint32_t)u[1];
                a[m][4 * v + 2] = (uint32_t)u[2]; a[m][4 * v + 3] = (uint32_t)u[3];
            }
    }

    int acc[R][MS];
#pragma unroll
    for (int r = 0; r < R; r++) {
#pragma unroll
        for (int m = 0; m < MS; m++) acc[r][m] = 0;
        if (live) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const uint32_t word = c == 0 ? w[r].x : c == 1 ? w[r].y : c == 2 ? w[r].z : w[r].w;
                const uint2 e0 = lut[0][word & 255u];
                const uint2 e1 = lut[1][(word >> 8) & 255u];
                const uint2 e2 = lut[2][(word >> 16) & 255u];
                const uint2 e3 = lut[3][word >> 24];
                const int d[5] = {(int)e0.x, (int)(e0.y | e1.x), (int)(e1.y | e2.x), (int)(e2.y | e3.x), (int)e3.y};
#pragma unroll
                for (int m = 0; m < MS; m++) {
                    int t = acc[r][m];
#pragma unroll
                    for (int i = 0; i < 5; i++) t = __builtin_amdgcn_sdot4(d[i], (int)a[m][5 * c + i], t, false);
                    acc[r][m] = t;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < MS; m++) {
            const int s = row16_sum(acc[r][m]);
            if ((tid & 15) == 0) part[r][m][tid >> 4] = s;
        }
    __syncthreads();
    if (tid < R * MS) {
        const int r = tid / MS, m = tid % MS;
        const int64_t n = n0 + r;
        int sum = 0;
#pragma unroll
        for (int x = 0; x < T / 16; x++) sum += part[r][m][x];
        // INT4 codes entered as 16 * q; the weights are plain trits
        if (m < M && n < N) store_y<YT>(Y + m * N + n, rescale(sum >> (BITS == 8 ? 0 : 4), xs[m], *alpha_p));
    }
}

template <int BITS, int MS, typename YT>
hipError_t launch_b3_t(const uint8_t* A, const float* xs, int64_t M, int64_t K, const uint8_t* W3,
                       const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    const int vpr = (int)((K + 79) / 80);
    const dim3 grid((unsigned)((N + kB3Rows - 1) / kB3Rows));
    switch ((vpr + 63) / 64) {
        case 1: hipLaunchKernelGGL((gemv_base3_kernel<BITS, MS, 64, kB3Rows, YT>), grid, dim3(64), 0, s, A, xs, (int)M, (int)K, vpr, W3, alpha, N, Y); break;
        case 2: hipLaunchKernelGGL((gemv_base3_kernel<BITS, MS, 128, kB3Rows, YT>), grid, dim3(128), 0, s, A, xs, (int)M, (int)K, vpr, W3, alpha, N, Y); break;
        default: hipLaunchKernelGGL((gemv_base3_kernel<BITS, MS, 256, kB3Rows, YT>), grid, dim3(256), 0, s, A, xs, (int)M, (int)K, vpr, W3, alpha, N, Y); break;
    }
    return hipGetLastError();
}

template <int BITS, typename YT>
hipError_t launch_b3_m(const uint8_t* A, const float* xs, int64_t M, int64_t K, const uint8_t* W3,
                       const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    if (M == 1) return launch_b3_t<BITS, 1, YT>(A, xs, M, K, W3, alpha, N, Y, s);
    if (M == 2) return launch_b3_t<BITS, 2, YT>(A, xs, M, K, W3, alpha, N, Y, s);
    return launch_b3_t<BITS, 4, YT>(A, xs, M, K, W3, alpha, N, Y, s);
}

}  // namespace

int64_t base3_row_bytes(int64_t K) { return 16 * ((K + 79) / 80); }

hipError_t launch_pack_base3(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W3, hipStream_t s) {
    const int vpr = (int)((K + 79) / 80);
    const int64_t total = N * vpr;
    hipLaunchKernelGGL(pack_base3_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       (const uint32_t*)W_packed, N, K, vpr, (uint4*)W3);
    return hipGetLastError();
}

// M in [1, 4], K % 16 == 0 and K <= 16384 (at most 256 vectors per row).
hipError_t launch_gemv_base3(const void* codes, const float* xscale, int act_bits, int64_t M, int64_t K,
                             const uint8_t* W3, const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s) {
    const uint8_t* A = (const uint8_t*)codes;
    if (act_bits == 8)
        return y_dtype == HBL_F32 ? launch_b3_m<8, float>(A, xscale, M, K, W3, alpha, N, (float*)Y, s)
                                  : launch_b3_m<8, uint16_t>(A, xscale, M, K, W3, alpha, N, (uint16_t*)Y, s);
    return y_dtype == HBL_F32 ? launch_b3_m<4, float>(A, xscale, M, K, W3, alpha, N, (float*)Y, s)
                              : launch_b3_m<4, uint16_t>(A, xscale, M, K, W3, alpha, N, (uint16_t*)Y, s);
}

}  // namespace hbl
