// hbl_device.h -- device-side helpers shared by the gfx950 kernels of libhbl.
// Internal header: not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hbl.h"

#define HBL_DEVINL __device__ __forceinline__

namespace hbl {

constexpr int kWave = 64;

// fp32 nearest to sqrt(7): bit pattern 0x402953FD (2.64575124f).
HBL_DEVINL float sqrt7_f32() { return __uint_as_float(0x402953FDu); }

HBL_DEVINL float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
HBL_DEVINL float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
HBL_DEVINL uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- raw buffer resources ----
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads whose offset falls
// outside return zeros and stores there are dropped, so tile edges need no
// branches (branch-free loads also let the compiler keep several loads in
// flight with exact vmcnt waits).  Ranges are clamped to 2^31 - 16 bytes.
HBL_DEVINL __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)lim, 0x00020000);
}
HBL_DEVINL uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- activation codes in the decode tile layout ----
// For the decode GEMM (up to 64 tokens), hbl_forward writes the codes tiled so
// that every wave instruction of the GEMM reads 1 KiB of consecutive bytes.
// Tokens are grouped in tiles of 16 rows and K in super-steps of 256 k
// (SSB = 32*BITS bytes per row).  Block (tile t, super-step ss) is 16 * SSB
// bytes at (t * K/256 + ss) * 16 * SSB; inside it, 16-byte chunk v*64 + g*16 + r
// holds bytes [g*SSB/4 + 16v, +16) of row r's super-step (g = 0..3 is the
// lane group of the 16x16x64 MFMA operand, v = 0 .. SSB/64 - 1).
template <int BITS>
HBL_DEVINL int64_t dec_tile_row_base(int64_t m, int64_t K) {
    constexpr int64_t SSB = 32 * BITS;
    return (m / 16) * (K / 256) * 16 * SSB + (m % 16) * 16;
}
template <int BITS>
HBL_DEVINL int dec_tile_offset(int kb) {  // kb: byte index of the code inside its row (>= 0)
    constexpr int SSB = 32 * BITS, Q = SSB / 4;
    const int rem = kb % SSB;
    return (kb / SSB) * 16 * SSB + ((rem % Q) / 16 * 64 + rem / Q * 16) * 16 + kb % 16;
}

// ---- INT4 codes as FP6 E3M2 for the FP6 x FP4 prefill GEMM ----
// The gfx950 matrix cores multiply FP6 by FP4 at twice the INT8 rate, and
// every INT4 code in [-8, 7] is exact in FP6 E3M2 (1 sign, 3 exponent bits
// with bias 3, 2 mantissa bits); a ternary weight is exact in FP4 E2M1.
// Code k of a row in natural order is the 6-bit field at bit 6k of a bit
// string, so 128 codes (one GEMM K step) are 96 bytes.  Inside a step, the 32
// codes k = 64s + 32h + j (j = 0..31) form one MFMA operand of 24 bytes; its
// first 16 bytes are stored as 16-byte chunk 2s + h of the step and its last
// 8 bytes as half s of chunk 4 + h, so that every lane reads one 16-byte and
// one 8-byte piece.  A row is K*3/4 bytes.
// Across rows the codes are grouped in bands of kF6Band rows (the GEMM's
// block height).  In a band of R rows (R = kF6Band except in the last band),
// K step s of all R rows is one block of R*96 bytes, row r of the band at
// byte 96r, so that every LDS-direct load of the GEMM reads 1 KiB of
// consecutive bytes.  Inside a row's 96 bytes the 16-byte chunks are stored
// in the GEMM's LDS order (bank-conflict-free reads): in rows with bit 3 of
// the row index set, chunk L sits at L ^ 1 (chunks 0..3) or 4 + ((L - 4) ^ 1)
// (chunks 4, 5).  The M*K*3/4 bytes are private to the FP6 x FP4 GEMM.
enum { kCodesRowMajor = 0, kCodesDecTiled = 1, kCodesFp6 = 2 };
constexpr int kF6Band = 256;

// ---- FP4 E2M1 weights (the library's W4 format, include/hbl.h) ----
// Weight rows in bands of kF4Band (the FP6 x FP4 GEMM's block width); in a
// band of R rows, K step s (128 weights, 64 bytes per row) of all R rows is
// one block of R*64 bytes, row r at byte 64r; inside a row's 64 bytes the
// 16-byte chunk c (weights 32c .. 32c+31) sits at c ^ ((r >> 2) & 3), the
// GEMM's LDS order; weight k at nibble k, low nibble first.  K % 128 == 0.
constexpr int kF4Band = 256;
// byte offset of the 8 bytes holding weights k .. k+15 (k % 16 == 0) of row n
HBL_DEVINL int64_t fp4_byte_offset(int64_t n, int64_t k, int64_t N, int64_t K) {
    const int64_t n0 = n - n % kF4Band;
    const int64_t R = N - n0 < kF4Band ? N - n0 : kF4Band;
    const int64_t r = n - n0, s = k / 128, c = (k % 128) / 32, h = (k % 32) / 16;
    return n0 * (K / 2) + (s * R + r) * 64 + ((c ^ ((r >> 2) & 3)) * 16) + 8 * h;
}
// Where row `row` of an M x K FP6 code matrix goes: its 96 bytes of K step s
// start at base + s * stride; swz = 1 where the chunks are swapped.
struct Fp6RowPlace {
    int64_t base;
    int64_t stride;
    int swz;
};
HBL_DEVINL Fp6RowPlace fp6_row_place(int64_t row, int64_t M, int64_t K) {
    const int64_t m0 = row - row % kF6Band;
    const int64_t R = M - m0 < kF6Band ? M - m0 : kF6Band;
    return Fp6RowPlace{m0 * (K * 3 / 4) + (row - m0) * 96, R * 96, (int)((row >> 3) & 1)};
}

// ---- wave / block reductions (fixed butterfly order: deterministic) ----
HBL_DEVINL float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
HBL_DEVINL float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}
HBL_DEVINL double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Block-wide reductions for NT threads (NT a multiple of 64).  `scratch` must
// hold NT/64 values of the reduced type; the result is returned to every
// thread.  Two barriers.
template <int NT>
HBL_DEVINL float block_sum_f32(float v, float* scratch) {
    v = wave_sum_f32(v);
    if constexpr (NT == kWave) return v;
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) r += scratch[i];
    __syncthreads();
    return r;
}
template <int NT>
HBL_DEVINL float block_max_f32(float v, float* scratch) {
    v = wave_max_f32(v);
    if constexpr (NT == kWave) return v;
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) r = fmaxf(r, scratch[i]);
    __syncthreads();
    return r;
}
template <int NT>
HBL_DEVINL double block_sum_f64(double v, double* scratch) {
    v = wave_sum_f64(v);
    if constexpr (NT == kWave) return v;
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int i = 0; i < NT / kWave; i++) r += scratch[i];
    __syncthreads();
    return r;
}

}  // namespace hbl

// ---- launchers implemented in the kernel translation units ----
namespace hbl {
hipError_t launch_weight_quant(const void* W, int w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                               float* alpha, double* partial, int n_partial, hipStream_t s);
int weight_partial_count(int64_t count);
// elements per partial-sum block (a multiple of 4096)
int64_t weight_partial_slice(int64_t count);
// the second of the two weight launches alone: alpha from the partial sums, then the 2-bit words
hipError_t launch_weight_pack(const void* W, int w_dtype, int64_t N, int64_t K, float eps, uint8_t* W_packed,
                              float* alpha, const double* partial, int n_partial, hipStream_t s);
// the first of the two weight launches alone: partial |W| sums into `partial`
hipError_t launch_weight_partial(const void* W, int w_dtype, int64_t count, double* partial, int n_partial,
                                 hipStream_t s);

// Activation quantisation of M rows and one half of the weight
// ternarisation in one launch: blocks [0, M) quantise rows, the rest either
// write the n_partial partial |W| sums into partial_out (partial_out not
// null; the packing follows with launch_weight_pack) or pack weight groups
// from the partial sums of an earlier launch_weight_partial.
hipError_t launch_act_and_pack(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                               const hbl_config& cfg, void* codes, float* xscale, const void* W, int w_dtype,
                               int64_t NK, float w_eps, const double* partial, double* partial_out, int n_partial,
                               uint8_t* W_packed,
                               float* alpha, hipStream_t s, int layout = kCodesRowMajor);  // K <= 2048

// layout: kCodesRowMajor (the ABI's), kCodesDecTiled, or kCodesFp6 (INT4, K >= 512)
hipError_t launch_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                            const hbl_config& cfg, void* codes, float* xscale, float* z_debug, float* s_debug,
                            hipStream_t s, int layout = kCodesRowMajor);

hipError_t launch_gemm(const void* codes, const float* xscale, int act_bits, int64_t M, int64_t K,
                       const uint8_t* W_packed, const float* alpha, int64_t N, void* Y, int y_dtype,
                       hipStream_t s, bool dec_tiled = false);
// FP6 x FP4 prefill GEMM (INT4 activation codes only): codes in the FP6
// layout above, weights as FP4 E2M1 nibbles in the FP4 layout above.  Same
// results as launch_gemm, bit for bit.
bool gemm_f6f4_eligible(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_f6f4(const uint8_t* codes6, const float* xscale, int64_t M, int64_t K, const uint8_t* W4,
                            const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s);
// 2-bit packed ternary weights -> FP4 E2M1 nibbles (W4 as above; K % 128 == 0)
hipError_t launch_weights_to_fp4(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W4, hipStream_t s);
// The layer's straight-through backward: dX (fp32 [M][K]) and, when dW is not
// null, dW (fp32 [N][K]); K a power of two in [512, 32768]; ws holds
// backward_ws_bytes(M, K, N, act_bits, dW != nullptr).
size_t backward_ws_bytes(int64_t M, int64_t K, int64_t N, int act_bits, bool want_dw);
hipError_t launch_backward(const void* dY, int dy_dtype, const void* X, int x_dtype, int64_t M, int64_t K,
                           const float* gain, const uint8_t* W_packed, const float* alpha, int64_t N,
                           const hbl_config& cfg, float* dX, float* dW, void* ws, hipStream_t s);
// per-(token, head) absmax quantisation of attention states to unsigned codes:
// V head vectors of D elements (fp32 or bf16) -> codes (D*bits/8 bytes each), d_out [V]
hipError_t launch_head_quant(const void* X, int x_dtype, int64_t V, int64_t D, int bits, float eps, uint8_t* codes,
                             float* d_out, hipStream_t s);
// base-3 weights (five per byte, rows of 16 * ceil(K/80) bytes)
int64_t base3_row_bytes(int64_t K);
hipError_t launch_pack_base3(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W3, hipStream_t s);
hipError_t launch_gemv_base3(const void* codes, const float* xscale, int act_bits, int64_t M, int64_t K,
                             const uint8_t* W3, const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s);
// true when launch_gemm runs the decode GEMM for this shape; the codes may
// then be in the decode tile layout (rows padded to a multiple of 16)
bool gemm_uses_decode_kernel(int64_t M, int64_t K);

// Sets the HIP error that hbl_last_hip_error() reports on this thread.
void record_hip_error(hipError_t e);
// Every check hbl_forward makes on its arguments except the workspace's
// (HBL_OK also for M == 0, which queues nothing).
hbl_status check_forward_args(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                              const uint8_t* W_packed, const float* alpha, int64_t N, const hbl_config* cfg,
                              const void* Y, int32_t y_dtype);

// The whole forward for M = kForwardSmallMaxM = 1 token and K a power of two
// in [1024, 16384], in one launch (codes and scale stay on chip).
constexpr int kForwardSmallMaxM = 1;
bool forward_small_eligible(int64_t M, int64_t K);
hipError_t launch_forward_small(const void* X, int x_dtype, int64_t M, int64_t K, const float* gain,
                                const hbl_config& cfg, const uint8_t* W_packed, const float* alpha, int64_t N,
                                void* Y, int y_dtype, hipStream_t s);
}  // namespace hbl
