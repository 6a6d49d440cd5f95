// gemm.hip -- INT8/INT4 activation codes x ternary 2-bit weights on the gfx950
// i8 matrix cores, int32 accumulation, fused rescale epilogue.
//
// The "新智元: 微软 BitNet v2" repost (section "原生4比特盘算") argues that dense
// low-bit compute, not sparsity, serves batched inference; the product
// acc[m][n] = sum_k q[m][k] W_q[n][k] is therefore a dense integer contraction
// and runs on MFMA.  The epilogue applies y = fp32(fp32(acc * xscale[m]) * alpha)
// (no bias: section "BitNet v2：原生4位激活").
//
// Operand unpacking (ternary weights to 64*w, INT4 codes to 16*q, both as
// int8) and the rescale are in int_dot.h.  For a given lane both MFMA
// operands hold the same k set, so the k order inside an operand does not
// matter to the result.
#include "int_dot.h"

namespace hbl {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

// Buffer stores: an offset outside the resource is dropped by the hardware.
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond every resource: store dropped

// ============================================================ prefill GEMM ==
// Block tile (64*TA) x (64*TB), K step 128, 4 waves in a 2 x 2 grid, each wave
// (32*TA) x (32*TB) = TA x TB MFMA 32x32x32 tiles.  LDS bandwidth is the
// binding resource of this kernel (the i8 MFMA itself sustains 4.2 POP/s even
// at one wave per SIMD with VALU work interleaved), and the fragment bytes a
// wave reads from LDS per MFMA are A/TB + W/TA (1 KiB and 256 B per 32x32
// fragment for INT8; 512 B and 256 B for INT4), so the default wave tile is
// 2 x 4 for large problems (>= 512 such tiles); small ones use 2 x 2 so that
// every CU still gets at least two blocks.  Both are built for two waves per
// SIMD (<= 256 registers).  Packed A and W tiles go global -> registers ->
// LDS (double buffered); kPF register buffers keep the global loads kPF-1 K
// steps ahead of their use.  Operands are unpacked in registers right before
// the MFMA.
//
// Tile order: blocks are dealt to the 8 XCDs round robin (block b -> XCD b%8);
// the kernel maps block b to tile (b%8)*T8 + b/8, so every XCD works on a
// contiguous band of M tiles and its L2 holds that band of A plus all of W.
constexpr int kBK = 128, kGemmThreads = 256, kPF = 2;

// k order inside a K step: 32-k MFMA step s of lane group g (lanes 32g..32g+31)
// takes the 16-k group 4g + s of the step, for both operands.  A lane's
// weight words for the whole step are then 16 contiguous bytes (one LDS read)
// and its INT4 codes 32 contiguous bytes.
template <int BITS, int BM>
struct ATile {
    static constexpr int row_bytes = BITS == 8 ? kBK : kBK / 2;  // bytes of one row per K step
    // padded LDS row (144 B INT8, 80 B INT4): 16 consecutive rows of 16-byte
    // reads at one column hit disjoint banks
    static constexpr int stride = row_bytes + 16;
    static constexpr int chunks = BM * row_bytes / 16;           // 16-byte chunks per tile
    static constexpr int per_thread = chunks / kGemmThreads;
    static constexpr int cpr = row_bytes / 16;                   // chunks per row
};
constexpr int kBRow = kBK / 4;        // 32 bytes of packed W per row and K step
constexpr int kBStride = kBRow + 16;  // 48 B: 16 consecutive columns of 16-byte reads hit disjoint banks

template <int BITS, int BM, int BN>
struct Regs {
    uint4 a[ATile<BITS, BM>::per_thread];
    uint4 b[BN * kBRow / 16 / kGemmThreads];
};

template <int BITS, typename YT, int TA, int TB>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_mfma_kernel(const uint8_t* __restrict__ A,
                                                                    const float* __restrict__ xscale, int64_t M,
                                                                    int64_t K, const uint8_t* __restrict__ Wp,
                                                                    const float* __restrict__ alpha_p, int64_t N,
                                                                    YT* __restrict__ Y, int tiles_n, int tiles_total) {
    constexpr int BM = 64 * TA, BN = 64 * TB;
    using AT = ATile<BITS, BM>;
    constexpr int kBPerThread = BN * kBRow / 16 / kGemmThreads;
    __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * AT::stride];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kBStride];
    __shared__ __attribute__((aligned(16))) float xs_tile[BM];  // per-token scales of this tile's rows (0 past M)

    // XCD-aware tile order (see above); falls back to linear order when the
    // tile count is not a multiple of 8.
    const int b = blockIdx.x;
    const int tile = (tiles_total % 8 == 0) ? (b % 8) * (tiles_total / 8) + b / 8 : b;
    const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t a_ld = K * BITS / 8;  // bytes per activation row
    const int64_t w_ld = K / 4;         // bytes per weight row
    const int KT = (int)(K / kBK);

    // rows past M (columns past N) lie outside these resources and load as zeros
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + m0 * a_ld, (M - m0) * a_ld);
    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(Wp + n0 * w_ld, (N - n0) * w_ld);
    auto load_tile = [&](Regs<BITS, BM, BN>& r, int kt) {
#pragma unroll
        for (int i = 0; i < AT::per_thread; i++) {
            const int q = tid + i * kGemmThreads;
            const int row = q / AT::cpr, c16 = q % AT::cpr;
            r.a[i] = buf_load16(a_rsrc, (uint32_t)(row * a_ld + kt * AT::row_bytes + c16 * 16));
        }
#pragma unroll
        for (int i = 0; i < kBPerThread; i++) {
            const int q = tid + i * kGemmThreads;
            const int row = q / (kBRow / 16), c16 = q % (kBRow / 16);
            r.b[i] = buf_load16(w_rsrc, (uint32_t)(row * w_ld + kt * kBRow + c16 * 16));
        }
    };
    auto store_tile = [&](const Regs<BITS, BM, BN>& r, int st) {
#pragma unroll
        for (int i = 0; i < AT::per_thread; i++) {
            const int q = tid + i * kGemmThreads;
            const int row = q / AT::cpr, c16 = q % AT::cpr;
            *reinterpret_cast<uint4*>(&As[st][row * AT::stride + c16 * 16]) = r.a[i];
        }
#pragma unroll
        for (int i = 0; i < kBPerThread; i++) {
            const int q = tid + i * kGemmThreads;
            const int row = q / (kBRow / 16), c16 = q % (kBRow / 16);
            *reinterpret_cast<uint4*>(&Bs[st][row * kBStride + c16 * 16]) = r.b[i];
        }
    };

    v16i acc[TA][TB];
#pragma unroll
    for (int i = 0; i < TA; i++)
#pragma unroll
        for (int j = 0; j < TB; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    const int lr = lane & 31;  // row (A) / column (W) inside a 32-wide MFMA tile
    const int lg = lane >> 5;  // which 16-k half of the 32-k MFMA step
    // Per K step a lane reads, for each of its TB columns, the four weight
    // words of its k groups (one 16-byte read), and for each of its TA rows
    // 16 bytes per MFMA step (INT8) or 32 bytes for all four (INT4).
    struct AFrag {
        v4i a[TA];
    };
    auto read_a = [&](AFrag& f, int st, int s) {
#pragma unroll
        for (int i = 0; i < TA; i++) {
            const int row = wm * 32 * TA + i * 32 + lr;
            const uint4 q = *reinterpret_cast<const uint4*>(&As[st][row * AT::stride + (BITS == 8 ? (4 * lg + s) * 16 : lg * 32 + s * 16)]);
            f.a[i][0] = (int)q.x; f.a[i][1] = (int)q.y; f.a[i][2] = (int)q.z; f.a[i][3] = (int)q.w;
        }
    };
    // Software pipeline: the A reads of step s+1 (INT8) or of the second
    // half (INT4) are issued before the MFMAs that precede them.
    auto compute = [&](int st) {
        uint4 wq[TB];
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int col = wn * 32 * TB + j * 32 + lr;
            wq[j] = *reinterpret_cast<const uint4*>(&Bs[st][col * kBStride + lg * 16]);
        }
        constexpr int kReads = BITS == 8 ? kBK / 32 : kBK / 64;  // A reads per K step
        AFrag f[2];
        read_a(f[0], st, 0);
#pragma unroll
        for (int s = 0; s < kBK / 32; s++) {
            const int rd = BITS == 8 ? s : s / 2;
            if ((BITS == 8 || s % 2 == 0) && rd + 1 < kReads) read_a(f[(rd + 1) & 1], st, rd + 1);
            const AFrag& cur = f[rd & 1];
            v4i bw[TB];
#pragma unroll
            for (int j = 0; j < TB; j++) {
                const uint32_t w = s == 0 ? wq[j].x : s == 1 ? wq[j].y : s == 2 ? wq[j].z : wq[j].w;
                bw[j] = unpack_w(w);
            }
#pragma unroll
            for (int i = 0; i < TA; i++) {
                v4i a;
                if constexpr (BITS == 8) a = cur.a[i];
                else a = (s & 1) ? unpack_a4((uint32_t)cur.a[i][2], (uint32_t)cur.a[i][3])
                                 : unpack_a4((uint32_t)cur.a[i][0], (uint32_t)cur.a[i][1]);
#pragma unroll
                for (int j = 0; j < TB; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bw[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    for (int r = tid; r < BM; r += kGemmThreads) {
        const __amdgpu_buffer_rsrc_t xs_rsrc = make_rsrc(xscale + m0, (M - m0) * 4);
        xs_tile[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xs_rsrc, r * 4, 0, 0));
    }

    // prologue: tiles 0..kPF-1 in flight, tile 0 in LDS stage 0
    Regs<BITS, BM, BN> R[kPF];
#pragma unroll
    for (int u = 0; u < kPF; u++) load_tile(R[u], min(u, KT - 1));
    store_tile(R[0], 0);
    __syncthreads();

    // Loads and LDS stores are unconditional (past the last tile they re-load
    // tile KT-1 and fill the idle LDS stage), so the compiler sees the same
    // number of loads in flight on every path and waits only for the oldest.
    for (int kt0 = 0; kt0 < KT; kt0 += kPF) {
#pragma unroll
        for (int u = 0; u < kPF; u++) {
            const int kt = kt0 + u;
            // R[(u+1)%kPF] holds tile kt+1; R[u] held tile kt (already in LDS)
            store_tile(R[(u + 1) % kPF], (kt + 1) & 1);
            load_tile(R[u], min(kt + kPF, KT - 1));
            if (kt < KT) compute(kt & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds column lr, rows 8*(r/4) + 4*lg + r%4 of each 32x32 tile.
    // Y is written through a buffer resource over this tile's rows: rows past M
    // fall outside it, columns past N start from an out-of-range offset; both
    // stores are dropped, so there are no per-element branches.  A lane's
    // offset is its base offset plus a row step that is uniform across the
    // wave; the four scales of rows 8q + 4lg .. +3 are one 16-byte LDS read.
    const float alpha = *alpha_p;
    const int rows_here = (int)min<int64_t>(BM, M - m0);
    const uint32_t row_bytes = (uint32_t)(N * (int64_t)sizeof(YT));  // <= 4 MiB (N <= 2^20)
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(Y + m0 * N, (int64_t)rows_here * row_bytes);
    const int row0 = wm * 32 * TA + 4 * lg;
#pragma unroll
    for (int j = 0; j < TB; j++) {
        const int64_t n = n0 + wn * 32 * TB + j * 32 + lr;
        const uint32_t lane_off = n < N ? (uint32_t)row0 * row_bytes + (uint32_t)(n * (int64_t)sizeof(YT)) : kDropOffset;
#pragma unroll
        for (int i = 0; i < TA; i++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 xs4 = *reinterpret_cast<const float4*>(&xs_tile[row0 + i * 32 + 8 * q]);
                const float xsr[4] = {xs4.x, xs4.y, xs4.z, xs4.w};
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; r++) y[r] = rescale(acc[i][j][4 * q + r] >> Shift<BITS>::value, xsr[r], alpha);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const uint32_t off = lane_off + (uint32_t)(i * 32 + 8 * q + r) * row_bytes;
                    if constexpr (sizeof(YT) == 4) {
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[r]), y_rsrc, (int)off, 0, 0);
                    } else if (r % 2 == 0) {
                        // hardware round-to-nearest-even pair conversion (same result as f32_to_bf16_bits)
                        const v2bf h = __builtin_convertvector((v2f){y[r], y[r + 1]}, v2bf);
                        const uint32_t hp = __builtin_bit_cast(uint32_t, h);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp & 0xFFFFu), y_rsrc, (int)off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp >> 16), y_rsrc, (int)(off + row_bytes), 0, 0);
                    }
                }
            }
        }
    }
}

// ============================================================ decode GEMM ==
// M <= 64 tokens: the packed weights (N*K/4 bytes) are the traffic, so the
// kernel is written to stream them at HBM rate.  One block of 8 waves per 16
// output columns; the waves split K.  A "super-step" covers 256 k: lane
// (n = lane%16, g = lane/16) loads one 16-byte vector of weight row n = 64
// trits k in [256*ss + 64*g, +64), so each instruction reads 16 rows x 64
// contiguous bytes.  Every wave issues all its weight vectors first (up to 16,
// 32 KiB per block in flight for K = 8192), then the activation codes in
// batches of at most 32 16-byte vectors per lane (they come from L2: every
// block reads the same codes).  MFMA 16x16x64 step d of a super-step takes,
// for lane group g, the 16-k chunk 256*ss + 64*g + 16*d; the activation
// operand uses the same chunk, so a lane's codes for one super-step are
// contiguous (32 bytes INT4, 64 bytes INT8).  The waves' int32 partial sums
// are added in LDS (exact) before the rescale.
constexpr int kDecWaves = 8, kDecThreads = kDecWaves * 64, kDecBN = 16, kDecMaxSS = 16, kDecSB = 4;

template <int BITS, int MT, typename YT>
__global__ __launch_bounds__(kDecThreads) void gemm_decode_kernel(const uint8_t* __restrict__ A,
                                                                  const float* __restrict__ xscale, int64_t M,
                                                                  int64_t K, const uint8_t* __restrict__ Wp,
                                                                  const float* __restrict__ alpha_p, int64_t N,
                                                                  YT* __restrict__ Y) {
    constexpr int kAVec = (BITS == 8 ? 64 : 32) / 16;              // 16-byte A vectors per super-step and tile
    constexpr int TG = (MT * kDecSB * kAVec <= 32) ? MT : 32 / (kDecSB * kAVec);  // token tiles per A batch
    __shared__ int red[kDecWaves][MT][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;  // weight column (W) / token row (A) inside the 16-wide tile
    const int g = lane >> 4;    // lane group: 64-k quarter of each super-step
    const int64_t n0 = (int64_t)blockIdx.x * kDecBN;
    const int64_t a_ld = K * BITS / 8;
    const int64_t w_ld = K / 4;
    const int SS = (int)(K / 256);  // super-steps in K
    const int per_wave = (SS + kDecWaves - 1) / kDecWaves;
    const int ss0 = wave * per_wave;
    const int cnt = max(0, min(SS, ss0 + per_wave) - ss0);

    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(Wp + n0 * w_ld, (N - n0) * w_ld);
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, M * a_ld);  // rows past M load as zeros
    const uint32_t w_lane = (uint32_t)(l16 * w_ld + g * 16);

    uint4 wv[kDecMaxSS];
#pragma unroll
    for (int u = 0; u < kDecMaxSS; u++)
        if (u < cnt) wv[u] = buf_load16(w_rsrc, w_lane + (uint32_t)(ss0 + u) * 64);

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) acc[t] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int sb = 0; sb < kDecMaxSS; sb += kDecSB) {
        if (sb < cnt) {
#pragma unroll
            for (int tg = 0; tg < MT; tg += TG) {
                uint4 aq[kDecSB][TG][kAVec];
#pragma unroll
                for (int u = 0; u < kDecSB; u++) {
                    const uint32_t k_byte = (uint32_t)(ss0 + sb + u) * (256 * BITS / 8) + g * (kAVec * 16);
#pragma unroll
                    for (int t = 0; t < TG; t++) {
                        const uint32_t a_lane = (uint32_t)(((tg + t) * 16 + l16) * a_ld) + k_byte;
#pragma unroll
                        for (int v = 0; v < kAVec; v++)
                            aq[u][t][v] = (sb + u < cnt) ? buf_load16(a_rsrc, a_lane + v * 16) : make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int u = 0; u < kDecSB; u++) {
                    if (sb + u < cnt) {
                        const uint32_t wd[4] = {wv[sb + u].x, wv[sb + u].y, wv[sb + u].z, wv[sb + u].w};
#pragma unroll
                        for (int d = 0; d < 4; d++) {
                            const v4i b = unpack_w(wd[d]);
#pragma unroll
                            for (int t = 0; t < TG; t++) {
                                v4i a;
                                if constexpr (BITS == 8) {
                                    const uint4 q = aq[u][t][d];
                                    a = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
                                } else {
                                    const uint4 q = aq[u][t][d >> 1];
                                    a = (d & 1) ? unpack_a4(q.z, q.w) : unpack_a4(q.x, q.y);
                                }
                                acc[tg + t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[tg + t], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int r = 0; r < 4; r++) red[wave][t][r][lane] = acc[t][r];
    __syncthreads();
    // wave w finishes token tiles t = w, w+8, ... (output: column l16, rows 4*g + r)
    const float alpha = *alpha_p;
    const int64_t n = n0 + l16;
    for (int t = wave; t < MT; t += kDecWaves) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            int sum = 0;
#pragma unroll
            for (int w = 0; w < kDecWaves; w++) sum += red[w][t][r][lane];
            const int64_t m = t * 16 + 4 * g + r;
            if (m < M && n < N) store_y<YT>(Y + m * N + n, rescale(sum >> Shift<BITS>::value, xscale[m], alpha));
        }
    }
}

// ======================================================= small-M GEMV ==
// M <= 4 tokens, K a power of two in [1024, 16384]: the GEMV routines of
// int_dot.h with 256 threads per 16 output columns, codes from global memory
// (loaded first, a few KiB from L2), then the weight stream.
constexpr int kGvThreads = 256;

template <int BITS, int LCPR, int MS, typename YT>
__global__ __launch_bounds__(kGvThreads) void gemv_small_kernel(const uint8_t* __restrict__ A,
                                                                const float* __restrict__ xscale, int M,
                                                                const uint8_t* __restrict__ Wp,
                                                                const float* __restrict__ alpha_p, int64_t N,
                                                                YT* __restrict__ Y) {
    using G = Gv<BITS, LCPR, MS, kGvThreads>;
    __shared__ typename G::Part part;
    const int64_t n0 = (int64_t)blockIdx.x * kGvRows;
    typename G::ARegs a;
    G::load_codes(A, M, a);
    typename G::WRegs w;
    G::load_w(Wp, n0, w);
    typename G::AOps av;
    G::unpack_codes(a, av);
    typename G::Acc acc;
    G::dot(w, av, acc);
    G::template finish<YT>(acc, part, M, xscale, *alpha_p, N, Y, n0);
}

template <int BITS, int MS, typename YT>
hipError_t launch_gemv_small(const uint8_t* A, const float* xscale, int64_t M, int64_t K, const uint8_t* Wp,
                             const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    const dim3 grid((unsigned)(N / kGvRows));
    switch (K) {
        case 1024: hipLaunchKernelGGL((gemv_small_kernel<BITS, 4, MS, YT>), grid, dim3(kGvThreads), 0, s, A, xscale, (int)M, Wp, alpha, N, Y); break;
        case 2048: hipLaunchKernelGGL((gemv_small_kernel<BITS, 5, MS, YT>), grid, dim3(kGvThreads), 0, s, A, xscale, (int)M, Wp, alpha, N, Y); break;
        case 4096: hipLaunchKernelGGL((gemv_small_kernel<BITS, 6, MS, YT>), grid, dim3(kGvThreads), 0, s, A, xscale, (int)M, Wp, alpha, N, Y); break;
        case 8192: hipLaunchKernelGGL((gemv_small_kernel<BITS, 7, MS, YT>), grid, dim3(kGvThreads), 0, s, A, xscale, (int)M, Wp, alpha, N, Y); break;
        default: hipLaunchKernelGGL((gemv_small_kernel<BITS, 8, MS, YT>), grid, dim3(kGvThreads), 0, s, A, xscale, (int)M, Wp, alpha, N, Y); break;
    }
    return hipGetLastError();
}

template <int BITS, typename YT>
hipError_t launch_typed(const uint8_t* A, const float* xscale, int64_t M, int64_t K, const uint8_t* Wp,
                        const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    if (M <= kGvMaxM && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0) {
        if (M == 1) return launch_gemv_small<BITS, 1, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
        if (M == 2) return launch_gemv_small<BITS, 2, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
        return launch_gemv_small<BITS, 4, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
    }
    if (M <= 64 && K % 256 == 0 && K / 256 <= kDecWaves * kDecMaxSS) {
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
    if (K % kBK != 0) return hipErrorInvalidValue;  // the C ABI only admits K % 128 == 0
    const int64_t big_tiles = ((M + 127) / 128) * ((N + 255) / 256);
    if (big_tiles >= 512) {
        const int tiles_n = (int)((N + 255) / 256);
        const int tiles_total = (int)big_tiles;
        hipLaunchKernelGGL((gemm_mfma_kernel<BITS, YT, 2, 4>), dim3(tiles_total), dim3(kGemmThreads), 0, s, A, xscale,
                           M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    } else {
        const int tiles_n = (int)((N + 127) / 128);
        const int tiles_total = tiles_n * (int)((M + 127) / 128);
        hipLaunchKernelGGL((gemm_mfma_kernel<BITS, YT, 2, 2>), dim3(tiles_total), dim3(kGemmThreads), 0, s, A, xscale,
                           M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    }
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
