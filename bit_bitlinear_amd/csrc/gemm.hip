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
#include "lds_dma.h"

namespace hbl {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

// ============================================================ prefill GEMM ==
// Block tile (64*TA) x (32*WGN*TB), K step 128, waves in a 2 x WGN grid, each
// wave (32*TA) x (32*TB) = TA x TB MFMA 32x32x32 tiles.  The fragment bytes a
// wave reads from LDS per MFMA are A/TB + W/TA (1 KiB and 256 B per 32x32
// fragment for INT8; 512 B and 256 B for INT4), so large problems (>= 512
// tiles of 128 x 256) use 4 waves with 2 x 4 wave tiles; smaller ones use 8
// waves with 2 x 2 wave tiles on the same 128 x 256 block.  Both run two
// waves per SIMD (<= 256 registers).  Operands are unpacked in registers
// right before the MFMA.
//
// Tile order: blocks are dealt to the 8 XCDs round robin (block b -> XCD b%8);
// the kernel maps block b to tile (b%8)*T8 + b/8, so every XCD works on a
// contiguous band of M tiles and its L2 holds that band of A plus all of W.
constexpr int kBK = 128, kGemmThreads = 256;

// Cache policy of the output stores of the prefill epilogues: non-temporal
// (bit 1) with device scope (bit 4).  Every block writes its whole tile at
// the end, all at about the same time, and nothing in the kernel reads Y
// back; streaming the writes past the caches took the 4096 x 2048 x 2048
// INT8 GEMM from 19.3-22.9 to 17.3-19.8 us (6-9% at 2048 x 4096 x 4096).
constexpr int kYStorePolicy = 2 | 16;

// k order inside a K step: 32-k MFMA step s of lane group g (lanes 32g..32g+31)
// takes the 16-k group 4g + s of the step, for both operands.  A lane's
// weight words for the whole step are then 16 contiguous bytes (one LDS read)
// and its INT4 codes 32 contiguous bytes.
//
// Loads: the packed tiles travel global -> LDS directly (buffer_load_dwordx4
// ... lds: lane l of a wave instruction writes its 16 bytes at LDS base +
// 16*l) through a ring of S stages, with no register staging and no LDS store
// instructions (about 10-15% faster than staging through registers).
// A wave instruction fills 1 KiB of LDS, so the LDS rows are unpadded; bank
// conflicts are avoided by an XOR swizzle of the 16-byte chunks instead,
// chosen so that 16 consecutive rows read at one logical chunk hit 16
// different 16-byte bank groups:
//   INT8 codes (128-byte rows): physical chunk = logical ^ ((row >> 1) & 7)
//   INT4 codes  (64-byte rows): physical chunk = logical ^ ((row >> 2) & 3)
//   weights     (32-byte rows): physical chunk = logical ^ ((row >> 3) & 1)
// The swizzle is applied on the global side (each lane fetches the logical
// chunk that belongs at its LDS position).  Out-of-range rows are zero-filled
// by the buffer range check, as for register loads.
template <int BITS, int TA, int TB, int WGN = 2>
struct DmaTile {
    static constexpr int NWAVES = 2 * WGN;                   // waves in a 2 x WGN grid
    static constexpr int BM = 64 * TA, BN = 32 * WGN * TB;
    static constexpr int a_row = BITS == 8 ? kBK : kBK / 2;  // code bytes per row and K step
    static constexpr int a_cpr = a_row / 16;                 // 16-byte chunks per code row
    static constexpr int a_bytes = BM * a_row;
    static constexpr int w_row = kBK / 4;                    // 32 bytes of packed W per row and K step
    static constexpr int w_bytes = BN * w_row;
    static constexpr int stage_bytes = a_bytes + w_bytes;
    static constexpr int a_inst = a_bytes / 1024 / NWAVES;   // 1 KiB DMA instructions per wave and K step
    static constexpr int w_inst = w_bytes / 1024 / NWAVES;
    static constexpr int inst = a_inst + w_inst;
    static_assert(a_bytes % (1024 * NWAVES) == 0 && w_bytes % (1024 * NWAVES) == 0,
                  "tile must split into whole wave instructions");
    static HBL_DEVINL int a_swz(int row) { return BITS == 8 ? (row >> 1) & 7 : (row >> 2) & 3; }
    static HBL_DEVINL int w_swz(int row) { return (row >> 3) & 1; }
};

template <int BITS, typename YT, int TA, int TB, int S, int WGN = 2>
__global__ __launch_bounds__(128 * WGN, TA == 1 ? 4 : 4 / WGN) void gemm_dma_kernel(const uint8_t* __restrict__ A,
                                                                   const float* __restrict__ xscale, int64_t M,
                                                                   int64_t K, const uint8_t* __restrict__ Wp,
                                                                   const float* __restrict__ alpha_p, int64_t N,
                                                                   YT* __restrict__ Y, int tiles_n, int tiles_total) {
    using DT = DmaTile<BITS, TA, TB, WGN>;
    constexpr int BM = DT::BM, BN = DT::BN;
    constexpr int NT = 64 * DT::NWAVES;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * DT::stage_bytes];
    __shared__ __attribute__((aligned(16))) float xs_tile[BM];  // per-token scales of this tile's rows (0 past M)

    const int b = blockIdx.x;
    const int tile = (tiles_total % 8 == 0) ? (b % 8) * (tiles_total / 8) + b / 8 : b;
    const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t a_ld = K * BITS / 8;  // bytes per activation row
    const int64_t w_ld = K / 4;         // bytes per weight row
    const int KT = (int)(K / kBK);

    const v4u a_desc = rsrc_words(A + m0 * a_ld, (M - m0) * a_ld);
    const v4u w_desc = rsrc_words(Wp + n0 * w_ld, (N - n0) * w_ld);

    // Per-lane global offsets (within one K step) of the chunks this lane
    // fetches in each of its DMA instructions; the K step adds kt * row bytes.
    uint32_t a_off[DT::a_inst], w_off[DT::w_inst];
#pragma unroll
    for (int u = 0; u < DT::a_inst; u++) {
        const int c = (wave * DT::a_inst + u) * 64 + lane;  // physical chunk index in the tile
        const int row = c / DT::a_cpr, p = c % DT::a_cpr;
        a_off[u] = (uint32_t)(row * a_ld + (p ^ DT::a_swz(row)) * 16);
    }
#pragma unroll
    for (int u = 0; u < DT::w_inst; u++) {
        const int c = (wave * DT::w_inst + u) * 64 + lane;
        const int row = c / 2, p = c % 2;
        w_off[u] = (uint32_t)(row * w_ld + (p ^ DT::w_swz(row)) * 16);
    }
    // LDS byte address of the ring (wave-uniform)
    const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    auto issue = [&](int kt, int st) {
        const uint32_t base = smem_addr + (uint32_t)(st * DT::stage_bytes);
#pragma unroll
        for (int u = 0; u < DT::a_inst; u++)
            lds_dma16(a_desc, __builtin_amdgcn_readfirstlane(base + (uint32_t)((wave * DT::a_inst + u) * 1024)),
                      a_off[u] + (uint32_t)(kt * DT::a_row));
#pragma unroll
        for (int u = 0; u < DT::w_inst; u++)
            lds_dma16(w_desc,
                      __builtin_amdgcn_readfirstlane(base + (uint32_t)(DT::a_bytes + (wave * DT::w_inst + u) * 1024)),
                      w_off[u] + (uint32_t)(kt * DT::w_row));
    };

    v16i acc[TA][TB];
#pragma unroll
    for (int i = 0; i < TA; i++)
#pragma unroll
        for (int j = 0; j < TB; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    const int lr = lane & 31;  // row (A) / column (W) inside a 32-wide MFMA tile
    const int lg = lane >> 5;  // lane group: takes the 16-k groups 4*lg .. 4*lg+3 of each K step
    struct AFrag {
        v4i a[TA];
    };
    auto read_a = [&](AFrag& f, const uint8_t* stage, int rd) {
#pragma unroll
        for (int i = 0; i < TA; i++) {
            const int row = wm * 32 * TA + i * 32 + lr;
            const int g = BITS == 8 ? 4 * lg + rd : 2 * lg + rd;  // logical 16-byte chunk
            const uint4 q = *reinterpret_cast<const uint4*>(stage + row * DT::a_row + ((g ^ DT::a_swz(row)) * 16));
            f.a[i][0] = (int)q.x; f.a[i][1] = (int)q.y; f.a[i][2] = (int)q.z; f.a[i][3] = (int)q.w;
        }
    };
    auto compute = [&](int st) {
        const uint8_t* stage = smem + st * DT::stage_bytes;
        uint4 wq[TB];
#pragma unroll
        for (int j = 0; j < TB; j++) {
            const int col = wn * 32 * TB + j * 32 + lr;
            wq[j] = *reinterpret_cast<const uint4*>(stage + DT::a_bytes + col * DT::w_row + ((lg ^ DT::w_swz(col)) * 16));
        }
        constexpr int kReads = BITS == 8 ? kBK / 32 : kBK / 64;  // A reads per K step
        AFrag f[2];
        read_a(f[0], stage, 0);
#pragma unroll
        for (int s = 0; s < kBK / 32; s++) {
            const int rd = BITS == 8 ? s : s / 2;
            if ((BITS == 8 || s % 2 == 0) && rd + 1 < kReads) read_a(f[(rd + 1) & 1], stage, rd + 1);
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

    // The per-token scales of the tile's rows (0 past M) are loaded into
    // registers first and written to LDS only for the epilogue, so their
    // latency hides behind the main loop instead of delaying the first loads.
    static_assert(BM <= NT, "one scale per thread");
    float xs_r = 0.f;
    if (tid < BM) {
        const __amdgpu_buffer_rsrc_t xs_rsrc = make_rsrc(xscale + m0, (M - m0) * 4);
        xs_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xs_rsrc, tid * 4, 0, 0));
    }

    // prologue: K steps 0..S-2 in flight (past the last step the loads repeat
    // step KT-1, so every wave always has the same number in flight)
#pragma unroll
    for (int u = 0; u < S - 1; u++) issue(min(u, KT - 1), u);
    for (int kt = 0; kt < KT; kt++) {
        wait_vmcnt<(S - 2) * DT::inst>();  // this wave's loads of step kt have landed
        barrier_no_wait();                 // ... and every wave's; stage (kt-1)%S is free
        issue(min(kt + S - 1, KT - 1), (kt + S - 1) % S);
        compute(kt % S);
    }
    wait_vmcnt<0>();  // no LDS-direct load may still be in flight when the block ends
    if (tid < BM) xs_tile[tid] = xs_r;
    __syncthreads();
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
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[r]), y_rsrc, (int)off, 0, kYStorePolicy);
                    } else if (r % 2 == 0) {
                        // hardware round-to-nearest-even pair conversion (same result as f32_to_bf16_bits)
                        const v2bf h = __builtin_convertvector((v2f){y[r], y[r + 1]}, v2bf);
                        const uint32_t hp = __builtin_bit_cast(uint32_t, h);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp & 0xFFFFu), y_rsrc, (int)off, 0, kYStorePolicy);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp >> 16), y_rsrc, (int)(off + row_bytes), 0, kYStorePolicy);
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
// With NB = 2 a block covers 32 columns: every activation operand feeds two
// MFMAs, which halves the activation codes read from L2 (the dominant
// traffic at 17-64 tokens); the weight vectors per wave double, so this form
// is used for K <= 8192 (at most MAXSS = 4 super-steps per wave), and only
// when it still leaves >= 256 blocks (N >= 8192): with fewer blocks the
// weight stream loses more than the halved activation reads gain (measured:
// 48 x 2048 x 8192 INT8 11.4 -> 6.9 us; 64 x 8192 x 4096 INT4 13.9 -> 14.6 us).
// With row-major codes each activation instruction reads 16 rows x 64 (INT4:
// 32) contiguous bytes; with TILED the codes are in the decode tile layout of
// hbl_device.h (written so by the activation kernel) and every instruction
// reads 1 KiB of consecutive bytes (measured 64 x 8192 x 4096 INT4 13.7 ->
// 9.9 us).
constexpr int kDecWaves = 8, kDecThreads = kDecWaves * 64, kDecBN = 16, kDecMaxSS = 16, kDecSB = 4;

template <int BITS, int MT, typename YT, int NB, int MAXSS, bool TILED>
__global__ __launch_bounds__(kDecThreads) void gemm_decode_kernel(const uint8_t* __restrict__ A,
                                                                  const float* __restrict__ xscale, int64_t M,
                                                                  int64_t K, const uint8_t* __restrict__ Wp,
                                                                  const float* __restrict__ alpha_p, int64_t N,
                                                                  YT* __restrict__ Y) {
    constexpr int kAVec = (BITS == 8 ? 64 : 32) / 16;              // 16-byte A vectors per super-step and tile
    constexpr int TG = (MT * kDecSB * kAVec <= 32) ? MT : 32 / (kDecSB * kAVec);  // token tiles per A batch
    __shared__ int red[kDecWaves][NB][MT][4][64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;  // weight column (W) / token row (A) inside the 16-wide tile
    const int g = lane >> 4;    // lane group: 64-k quarter of each super-step
    const int64_t n0 = (int64_t)blockIdx.x * kDecBN * NB;
    const int64_t a_ld = K * BITS / 8;
    const int64_t w_ld = K / 4;
    const int SS = (int)(K / 256);  // super-steps in K
    const int per_wave = (SS + kDecWaves - 1) / kDecWaves;
    const int ss0 = wave * per_wave;
    const int cnt = max(0, min(SS, ss0 + per_wave) - ss0);

    const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(Wp + n0 * w_ld, (N - n0) * w_ld);
    // rows past M load as zeros (row-major) or as the unwritten padding rows of
    // the last tile (TILED); either way they reach only output rows >= M,
    // which are not stored
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A, (TILED ? (M + 15) / 16 * 16 : M) * a_ld);

    uint4 wv[NB][MAXSS];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const uint32_t w_lane = (uint32_t)((nb * kDecBN + l16) * w_ld + g * 16);
#pragma unroll
        for (int u = 0; u < MAXSS; u++)
            if (u < cnt) wv[nb][u] = buf_load16(w_rsrc, w_lane + (uint32_t)(ss0 + u) * 64);
    }

    v4i acc[NB][MT];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int t = 0; t < MT; t++) acc[nb][t] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int sb = 0; sb < MAXSS; sb += kDecSB) {
        if (sb < cnt) {
#pragma unroll
            for (int tg = 0; tg < MT; tg += TG) {
                uint4 aq[kDecSB][TG][kAVec];
#pragma unroll
                for (int u = 0; u < kDecSB; u++) {
                    constexpr uint32_t SSB = 256 * BITS / 8;  // bytes per row and super-step
                    const uint32_t ss = (uint32_t)(ss0 + sb + u);
#pragma unroll
                    for (int t = 0; t < TG; t++) {
                        // tile (tg + t) starts at byte 16 * a_ld in both layouts
                        const uint32_t a_lane =
                            TILED ? (uint32_t)((tg + t) * 16 * a_ld) + ss * 16 * SSB + lane * 16
                                  : (uint32_t)(((tg + t) * 16 + l16) * a_ld) + ss * SSB + g * (kAVec * 16);
#pragma unroll
                        for (int v = 0; v < kAVec; v++)
                            aq[u][t][v] = (sb + u < cnt) ? buf_load16(a_rsrc, a_lane + v * (TILED ? 1024 : 16))
                                                         : make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int u = 0; u < kDecSB; u++) {
                    if (sb + u < cnt) {
#pragma unroll
                        for (int d = 0; d < 4; d++) {
                            v4i bw[NB];
#pragma unroll
                            for (int nb = 0; nb < NB; nb++) {
                                const uint4 q = wv[nb][sb + u];
                                bw[nb] = unpack_w(d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w);
                            }
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
#pragma unroll
                                for (int nb = 0; nb < NB; nb++)
                                    acc[nb][tg + t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bw[nb], acc[nb][tg + t], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int r = 0; r < 4; r++) red[wave][nb][t][r][lane] = acc[nb][t][r];
    __syncthreads();
    // wave w finishes (column tile, token tile) pairs p = w, w+8, ... (output:
    // column l16 of the tile, rows 4*g + r)
    const float alpha = *alpha_p;
    for (int p = wave; p < NB * MT; p += kDecWaves) {
        const int nb = p / MT, t = p % MT;
        const int64_t n = n0 + nb * kDecBN + l16;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            int sum = 0;
#pragma unroll
            for (int w = 0; w < kDecWaves; w++) sum += red[w][nb][t][r][lane];
            const int64_t m = t * 16 + 4 * g + r;
            if (m < M && n < N) store_y<YT>(Y + m * N + n, rescale(sum >> Shift<BITS>::value, xscale[m], alpha));
        }
    }
}

// ======================================================= small-M GEMV ==// ======================================================= small-M GEMV ==
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

// Ring depth: 3 stages (loads two K steps ahead) for the 4-wave blocks, where
// a fourth 24 KiB stage would leave room for one block per CU instead of two;
// 4 stages for the 8-wave blocks, which run one block per CU (3-6% faster than
// 3 stages at 4096 x 2048 x 2048 INT8 and INT4 and at 2048 x 4096 x 4096).
constexpr int kDmaStages = 3;
constexpr int kDmaStages8w = 4;

bool gemv_small_shape(int64_t M, int64_t K) {
    return M <= kGvMaxM && K >= 1024 && K <= 16384 && (K & (K - 1)) == 0;
}

template <int BITS, typename YT, bool TILED>
hipError_t launch_decode(const uint8_t* A, const float* xscale, int64_t M, int64_t K, const uint8_t* Wp,
                         const float* alpha, int64_t N, YT* Y, hipStream_t s) {
    if (M > 16 && K / 256 <= kDecWaves * 4 && N >= 256 * 2 * kDecBN) {
        const dim3 grid((unsigned)((N + 2 * kDecBN - 1) / (2 * kDecBN)));
        if (M <= 32)
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, 2, YT, 2, 4, TILED>), grid, dim3(kDecThreads), 0, s, A,
                               xscale, M, K, Wp, alpha, N, Y);
        else
            hipLaunchKernelGGL((gemm_decode_kernel<BITS, 4, YT, 2, 4, TILED>), grid, dim3(kDecThreads), 0, s, A,
                               xscale, M, K, Wp, alpha, N, Y);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + kDecBN - 1) / kDecBN));
    if (M <= 16)
        hipLaunchKernelGGL((gemm_decode_kernel<BITS, 1, YT, 1, kDecMaxSS, TILED>), grid, dim3(kDecThreads), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y);
    else if (M <= 32)
        hipLaunchKernelGGL((gemm_decode_kernel<BITS, 2, YT, 1, kDecMaxSS, TILED>), grid, dim3(kDecThreads), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y);
    else
        hipLaunchKernelGGL((gemm_decode_kernel<BITS, 4, YT, 1, kDecMaxSS, TILED>), grid, dim3(kDecThreads), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y);
    return hipGetLastError();
}

template <int BITS, typename YT>
hipError_t launch_typed(const uint8_t* A, const float* xscale, int64_t M, int64_t K, const uint8_t* Wp,
                        const float* alpha, int64_t N, YT* Y, hipStream_t s, bool dec_tiled) {
    if (gemv_small_shape(M, K)) {
        if (M == 1) return launch_gemv_small<BITS, 1, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
        if (M == 2) return launch_gemv_small<BITS, 2, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
        return launch_gemv_small<BITS, 4, YT>(A, xscale, M, K, Wp, alpha, N, Y, s);
    }
    if (gemm_uses_decode_kernel(M, K))
        return dec_tiled ? launch_decode<BITS, YT, true>(A, xscale, M, K, Wp, alpha, N, Y, s)
                         : launch_decode<BITS, YT, false>(A, xscale, M, K, Wp, alpha, N, Y, s);
    if (dec_tiled) return hipErrorInvalidValue;  // the tile layout is only read by the decode GEMM
    if (K % kBK != 0) return hipErrorInvalidValue;  // the C ABI only admits K % 128 == 0
    const int64_t big_tiles = ((M + 127) / 128) * ((N + 255) / 256);
    if (big_tiles >= 512) {
        const int tiles_n = (int)((N + 255) / 256);
        const int tiles_total = (int)big_tiles;
        hipLaunchKernelGGL((gemm_dma_kernel<BITS, YT, 2, 4, kDmaStages>), dim3(tiles_total), dim3(kGemmThreads), 0, s, A, xscale,
                           M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    } else if (big_tiles >= 128) {
        // smaller problems: 128 x 256 blocks of 8 waves (2 x 4 grid of 64 x 64
        // wave tiles), one block and two waves per SIMD per CU; the code tile
        // in LDS serves twice as many columns as a 4-wave 128 x 128 block
        // (measured 3% faster at 4096 x 2048 x 2048)
        const int tiles_n = (int)((N + 255) / 256);
        const int tiles_total = tiles_n * (int)((M + 127) / 128);
        hipLaunchKernelGGL((gemm_dma_kernel<BITS, YT, 2, 2, kDmaStages8w, 4>), dim3(tiles_total), dim3(512), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    } else if constexpr (BITS == 8) {
        // fewer than 128 tiles of 128 x 256 (a few hundred tokens): 64-row
        // tiles, 8 waves of 32 x 64, up to two blocks per CU, so twice as
        // many CUs take part (measured 256 x 4096 x 4096: 26.3 -> 18.6 us)
        const int tiles_n = (int)((N + 255) / 256);
        const int tiles_total = tiles_n * (int)((M + 63) / 64);
        hipLaunchKernelGGL((gemm_dma_kernel<BITS, YT, 1, 2, kDmaStages8w, 4>), dim3(tiles_total), dim3(512), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    } else {
        // the same for INT4 codes (64-byte rows: a 64-row code tile is too
        // small for 8 waves' LDS-direct loads): 64 x 128 tiles of 4 waves
        const int tiles_n = (int)((N + 127) / 128);
        const int tiles_total = tiles_n * (int)((M + 63) / 64);
        hipLaunchKernelGGL((gemm_dma_kernel<BITS, YT, 1, 2, kDmaStages, 2>), dim3(tiles_total), dim3(256), 0, s, A,
                           xscale, M, K, Wp, alpha, N, Y, tiles_n, tiles_total);
    }
    return hipGetLastError();
}

// ===================================================== FP6 x FP4 GEMM ==
// INT4 codes x ternary weights on v_mfma_f32_32x32x64_f8f6f4 with the codes
// as FP6 E3M2 and the weights as FP4 E2M1 (formats in hbl_device.h): on gfx950
// this runs at twice the INT8 MFMA rate.  Every product is an integer and
// every partial sum is below 2^24 in magnitude (|acc| <= 8*K <= 2^18), so the
// fp32 accumulation is exact in any order and equals the INT8 path's int32
// accumulator; the epilogue applies the same two rounded products, so the
// outputs are the same bit for bit.
// Block 256 x 256, 8 waves in a 4 x 2 grid of 64 x 128 wave tiles (2 x 4 MFMA
// tiles of 32 x 32), K step 128 = two MFMA k-steps.  Per K step a row moves
// 96 bytes of codes and 64 bytes of weights global -> LDS directly (as in the
// INT8 kernel), through a ring of S stages of 40 KiB (S = 4 fills the 160 KiB
// of LDS; the per-token scales then reuse the ring after the main loop).
// Physical 16-byte chunk of logical chunk L of row r in LDS (bank-conflict-free
// 16-byte reads):
//   codes, 16-byte pieces (chunks 0..3): L ^ ((r >> 3) & 1)
//   codes, 8-byte pieces  (chunks 4, 5): 4 + ((L - 4) ^ ((r >> 3) & 1))
//   weights (chunks 0..3):               L ^ ((r >> 2) & 3)
// Both maps are their own inverse.  The activation kernel stores the codes
// already in this order, in blocks of one K step of a 256-row band (the FP6
// layout of hbl_device.h), and the FP4 weight format stores the weights the
// same way, so every load instruction copies 1 KiB of consecutive bytes.
// Against rows of 96 (64) bytes at the row stride of row-major layouts this
// made the GEMM 9-11% faster on the 3B-like shapes for the codes, and about
// 3% more for the weights.
//
// Main loop, software-pipelined: the LDS fragments of the next MFMA k-step
// are read while the current k-step's MFMAs run (scheduling barriers keep the
// compiler from sinking the reads next to their use; the reads are spread one
// between each two MFMAs), and a lane's two 8-byte
// code tails of a K step (chunks 4 + lh, both halves) come in one 16-byte
// read.  One block barrier per K step sits between the two k-steps: it
// publishes the next stage (each wave first waits for its own loads of it)
// and certifies that every wave has consumed the stage the new loads
// overwrite.  Measured against the unpipelined 3-stage loop (graph replay,
// 3B-like shapes): 8-10% faster; without any global loads the same loop runs
// at about half the matrix-core peak, so the LDS-direct loads and the LDS
// reads, not load latency, set the pace (a variant with the vmcnt waits
// removed was no faster).
constexpr int kF6ARow = 96, kF6WRow = 64;  // bytes per row and K step

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));


// Block BM x BN, WGM x WGN waves of (BM/WGM) x (BN/WGN), S-stage ring.
template <int BM, int BN, int WGM, int WGN, int S>
struct F6Tile {
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int TA = BM / WGM / 32, TB = BN / WGN / 32;  // 32 x 32 MFMA tiles per wave
    static constexpr int a_bytes = BM * kF6ARow, w_bytes = BN * kF6WRow, stage = a_bytes + w_bytes;
    static constexpr int a_inst = a_bytes / 1024 / NW, w_inst = w_bytes / 1024 / NW, inst = a_inst + w_inst;
    static constexpr bool xs_in_ring = S * stage + BM * 4 > 163840;  // scales reuse the ring
    static constexpr int lds_bytes = S * stage + (xs_in_ring ? 0 : BM * 4);
    static_assert(a_bytes % (1024 * NW) == 0 && w_bytes % (1024 * NW) == 0, "whole wave instructions");
    static_assert(BM <= NT, "one scale per thread");
    static_assert(S >= 3 && lds_bytes <= 163840, "ring depth");
};

// Tile order: blocks are dealt to the 8 XCDs round robin (block b -> XCD
// b % 8), so block b first takes index t = (b % 8) * T/8 + b / 8 (a contiguous
// range of T/8 tiles per XCD); inside that range groups of 4 tile rows walk
// the tile columns together, so the blocks resident on one XCD at a time
// share 4 bands of codes and a few bands of weights in its L2 (3-7% faster
// than walking whole tile rows on the 3B-like gate/up and QKV shapes).
HBL_DEVINL int f6_tile_of_block(int b, int tiles_n, int tiles_total) {
    if (tiles_total % 8 != 0) return b;
    const int t = (b % 8) * (tiles_total / 8) + b / 8;
    constexpr int G = 4;
    const int tiles_m = tiles_total / tiles_n;
    const int grp = t / (G * tiles_n), in = t % (G * tiles_n);
    const int rows = min(G, tiles_m - grp * G);
    return (grp * G + in % rows) * tiles_n + in / rows;
}

template <typename YT, int BM, int BN, int WGM, int WGN, int S>
__global__ __launch_bounds__(64 * WGM * WGN, 2) void gemm_f6f4_kernel(
    const uint8_t* __restrict__ A6, const float* __restrict__ xscale, int64_t M, int64_t K,
    const uint8_t* __restrict__ W4, const float* __restrict__ alpha_p, int64_t N, YT* __restrict__ Y, int tiles_n,
    int tiles_total, int stagger) {
    using T = F6Tile<BM, BN, WGM, WGN, S>;
    // De-phasing: every block of one wave of tiles reaches its epilogue at
    // the same moment and the output write then runs alone at HBM write
    // speed.  With many waves of tiles the first wave's blocks start
    // staggered by XCD, `stagger` x 64 cycles apart; the later blocks inherit
    // the offsets, so one XCD's epilogue overlaps the others' main loops
    // (3-5% on the 3B-like gate/up shape, 16 waves of tiles; nothing gained
    // with 6 or fewer, so the launcher passes 0 there).
    if (stagger > 0 && (int)blockIdx.x < 256) {
        const int n = (int)(blockIdx.x & 7) * stagger;
        for (int i = 0; i < n; i += 16) __builtin_amdgcn_s_sleep(16);
    }
    constexpr int TA = T::TA, TB = T::TB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::lds_bytes];
    float* const xs_tile = reinterpret_cast<float*>(smem + (T::xs_in_ring ? 0 : S * T::stage));

    const int tile = f6_tile_of_block(blockIdx.x, tiles_n, tiles_total);
    const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t a_ld = K * 3 / 4;  // bytes per code row
    const int64_t w_ld = K / 2;      // bytes per weight row
    const int KT = (int)(K / kBK);

    // codes: the tile's band of rows_a rows holds K step kt as one block of
    // rows_a * 96 bytes, already in LDS order (hbl_device.h), so each load
    // instruction copies 1 KiB of consecutive bytes.  Every K step's loads
    // get a buffer resource covering exactly that block: in a band of fewer
    // than BM rows the lanes past the block read zeros (they feed only output
    // rows that are not stored), and no load leaves the block.  (The scalar
    // soffset of a buffer load is not part of its range check, so the step
    // may not ride there: with the banded layout it is far larger than the
    // block, and a short last band would read past the end of its buffer.)
    static_assert(BM == kF6Band, "the FP6 code bands are the block height");
    const int rows_a = (int)min<int64_t>(BM, M - m0);
    const uint8_t* const a_band = A6 + m0 * a_ld;
    const int64_t a_blk = (int64_t)rows_a * kF6ARow;  // bytes of one K step's block
    // weights: the same for the FP4 layout's 256-row bands (blocks of one K
    // step, rows_w * 64 bytes, in LDS order)
    static_assert(BN == kF4Band, "the FP4 weight bands are the block width");
    const int rows_w = (int)min<int64_t>(BN, N - n0);
    const uint8_t* const w_band = W4 + n0 * w_ld;
    const int64_t w_blk = (int64_t)rows_w * kF6WRow;
    uint32_t a_off[T::a_inst], w_off[T::w_inst];
#pragma unroll
    for (int u = 0; u < T::a_inst; u++) a_off[u] = (uint32_t)(((wave * T::a_inst + u) * 64 + lane) * 16);
#pragma unroll
    for (int u = 0; u < T::w_inst; u++) w_off[u] = (uint32_t)(((wave * T::w_inst + u) * 64 + lane) * 16);
    const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
    // the K step moves the resources' (scalar) base; the per-lane offsets
    // stay fixed, and the LDS destinations are wave-uniform, computed in
    // scalar registers
    const uint32_t wave_s = __builtin_amdgcn_readfirstlane((uint32_t)wave);
    const uint32_t a_dst = __builtin_amdgcn_readfirstlane(smem_addr) + wave_s * (uint32_t)(T::a_inst * 1024);
    const uint32_t w_dst = __builtin_amdgcn_readfirstlane(smem_addr) + (uint32_t)T::a_bytes +
                           wave_s * (uint32_t)(T::w_inst * 1024);
    auto issue = [&](int kt, int st) {
        const uint32_t st_off = (uint32_t)(st * T::stage);
        const v4u a_desc = rsrc_words(a_band + kt * a_blk, a_blk);
        const v4u w_desc = rsrc_words(w_band + kt * w_blk, w_blk);
#pragma unroll
        for (int u = 0; u < T::a_inst; u++) lds_dma16(a_desc, a_dst + st_off + (uint32_t)(u * 1024), a_off[u]);
#pragma unroll
        for (int u = 0; u < T::w_inst; u++) lds_dma16(w_desc, w_dst + st_off + (uint32_t)(u * 1024), w_off[u]);
    };

    v16f acc[TA][TB];
#pragma unroll
    for (int i = 0; i < TA; i++)
#pragma unroll
        for (int j = 0; j < TB; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // per-lane LDS byte offsets inside a stage: lane (lr, lh) reads row / column
    // lr of each 32-wide MFMA tile, k 32*lh .. +31 of each 64-k MFMA step
    const int lr = lane & 31;
    const int lh = lane >> 5;
    // The code swizzle of row r = wm*32*TA + i*32 + lr depends only on bit 3
    // of lr, and the weight swizzle of column c = wn*32*TB + j*32 + lr only on
    // bits 2-3 of lr, so every fragment offset is a per-lane base plus a
    // constant: codes a_lane + i*32 rows + 32 bytes per k-step (+64 for the
    // 8-byte pieces), weights w_lane[k-step] + j*32 rows.  The LDS reads then
    // take the constants as immediate offsets instead of an address add each.
    const int a_lane = (wm * 32 * TA + lr) * kF6ARow + 16 * (lh ^ ((lr >> 3) & 1));
    int w_lane[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; s2++)
        w_lane[s2] = T::a_bytes + (wn * 32 * TB + lr) * kF6WRow + (((2 * s2 + lh) ^ ((lr >> 2) & 3)) * 16);
    // fragments of the two k-steps of a K step (fa0/fw0: k-step 0, fa1/fw1:
    // k-step 1) and the code tails of two consecutive K steps
    uint4 fa0[TA], fw0[TB], fa1[TA], fw1[TB], ta[TA], tb[TA];
#define HBL_F6_READ(FA, FW, ST, S2)                                                                          \
    {                                                                                                        \
        _Pragma("unroll") for (int i = 0; i < TA; i++)                                                      \
            FA[i] = *reinterpret_cast<const uint4*>((ST) + a_lane + (i * 32 * kF6ARow + 32 * (S2)));          \
        _Pragma("unroll") for (int j = 0; j < TB; j++)                                                      \
            FW[j] = *reinterpret_cast<const uint4*>((ST) + w_lane[S2] + j * 32 * kF6WRow);                    \
    }
#define HBL_F6_TAIL(TL, ST) \
    { _Pragma("unroll") for (int i = 0; i < TA; i++) TL[i] = *reinterpret_cast<const uint4*>((ST) + a_lane + (i * 32 * kF6ARow + 64)); }
    // formats: 3 = FP6 E3M2 (codes), 4 = FP4 E2M1 (weights); unscaled
#define HBL_F6_MFMA(FA, FW, TL, S2)                                                                          \
    {                                                                                                        \
        _Pragma("unroll") for (int i = 0; i < TA; i++) {                                                    \
            const v8i a = v8i{(int)FA[i].x, (int)FA[i].y, (int)FA[i].z, (int)FA[i].w,                        \
                              (int)((S2) ? TL[i].z : TL[i].x), (int)((S2) ? TL[i].w : TL[i].y), 0, 0};       \
            _Pragma("unroll") for (int j = 0; j < TB; j++) {                                                \
                const v8i w = v8i{(int)FW[j].x, (int)FW[j].y, (int)FW[j].z, (int)FW[j].w, 0, 0, 0, 0};       \
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, w, acc[i][j], 3, 4, 0, 0, 0, 0); \
            }                                                                                                \
        }                                                                                                    \
    }
    // One K step kt, entered with fa0/fw0 = k-step 0 of kt and TL = its tails;
    // leaves fa0/fw0 = k-step 0 of kt + 1 and TN = its tails.  Past the last
    // step the reads fetch a stage whose contents are not used.
    // one LDS read between consecutive MFMAs, rather than the reads in a
    // burst, keeps the LDS queue short (3-4% faster on the 3B-like shapes)
#define HBL_F6_INTERLEAVE(NREADS)                                                                            \
    {                                                                                                        \
        _Pragma("unroll") for (int q = 0; q < (NREADS); q++) {                                              \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* one LDS read */                           \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* one MFMA */                               \
        }                                                                                                    \
    }
#define HBL_F6_STEP(KT_, TL, TN)                                                                             \
    {                                                                                                        \
        const int kk = (KT_);                                                                                \
        const uint8_t* stage = smem + (kk % S) * T::stage;                                                   \
        HBL_F6_READ(fa1, fw1, stage, 1);                                                                     \
        HBL_F6_MFMA(fa0, fw0, TL, 0);                                                                        \
        HBL_F6_INTERLEAVE(TA + TB);                                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                                   \
        wait_vmcnt<(S - 3) * T::inst>(); /* this wave's loads of step kk + 1 have landed */                  \
        barrier_no_wait();               /* ... every wave's; stage (kk - 1) % S is consumed */              \
        issue(min(kk + S - 1, KT - 1), (kk + S - 1) % S);                                                    \
        const uint8_t* nstage = smem + ((kk + 1) % S) * T::stage;                                            \
        HBL_F6_READ(fa0, fw0, nstage, 0);                                                                    \
        HBL_F6_TAIL(TN, nstage);                                                                             \
        HBL_F6_MFMA(fa1, fw1, TL, 1);                                                                        \
        HBL_F6_INTERLEAVE(2 * TA + TB);                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                                   \
    }

    float xs_r = 0.f;  // scale of row tid (0 past M), used only in the epilogue
    if (tid < BM) {
        const __amdgpu_buffer_rsrc_t xs_rsrc = make_rsrc(xscale + m0, (M - m0) * 4);
        xs_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xs_rsrc, tid * 4, 0, 0));
    }
    // prologue: K steps 0..S-2 in flight (past the last step the loads repeat
    // step KT-1, so every wave always has the same number in flight)
#pragma unroll
    for (int u = 0; u < S - 1; u++) issue(min(u, KT - 1), u);
    wait_vmcnt<(S - 2) * T::inst>();  // this wave's loads of step 0 have landed
    barrier_no_wait();
    HBL_F6_READ(fa0, fw0, smem, 0);
    HBL_F6_TAIL(ta, smem);
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {  // two K steps per pass, so the tail registers alternate
        HBL_F6_STEP(kt, ta, tb);
        HBL_F6_STEP(kt + 1, tb, ta);
    }
    if (kt < KT) HBL_F6_STEP(kt, ta, tb);
#undef HBL_F6_STEP
#undef HBL_F6_INTERLEAVE
#undef HBL_F6_MFMA
#undef HBL_F6_TAIL
#undef HBL_F6_READ
    wait_vmcnt<0>();  // no LDS-direct load may still be in flight when the block ends
    __syncthreads();  // every wave is done with the ring (the scales may reuse it)
    if (tid < BM) xs_tile[tid] = xs_r;
    __syncthreads();

    // epilogue as in the INT8 kernel: lane holds column lr, rows 8*(r/4) + 4*lh + r%4 of each tile
    const float alpha = *alpha_p;
    const int rows_here = (int)min<int64_t>(BM, M - m0);
    const uint32_t row_bytes = (uint32_t)(N * (int64_t)sizeof(YT));
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(Y + m0 * N, (int64_t)rows_here * row_bytes);
    const int row0 = wm * 32 * TA + 4 * lh;
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
                for (int r = 0; r < 4; r++) {
                    const float t = acc[i][j][4 * q + r] * xsr[r];  // two separately rounded products
                    y[r] = t * alpha;
                }
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const uint32_t off = lane_off + (uint32_t)(i * 32 + 8 * q + r) * row_bytes;
                    if constexpr (sizeof(YT) == 4) {
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[r]), y_rsrc, (int)off, 0, kYStorePolicy);
                    } else if (r % 2 == 0) {
                        const v2bf h = __builtin_convertvector((v2f){y[r], y[r + 1]}, v2bf);
                        const uint32_t hp = __builtin_bit_cast(uint32_t, h);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp & 0xFFFFu), y_rsrc, (int)off, 0, kYStorePolicy);
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(hp >> 16), y_rsrc, (int)(off + row_bytes), 0, kYStorePolicy);
                    }
                }
            }
        }
    }
}

// Shape used: 256 x 256 blocks of 8 waves (4 x 2 grid of 64 x 128 wave tiles), 4 stages.
constexpr int kF6BM = 256, kF6BN = 256, kF6WGM = 4, kF6WGN = 2, kF6Stages = 4;

// 2-bit packed weights -> FP4 E2M1: one 32-bit word (16 weights; weight e of
// the group at bits 8*(e%4) + 2*(e/4)) -> 8 bytes (weight e at nibble e), put
// at its place in the FP4 layout (fp4_byte_offset).
// The 2-bit code c (00 = 0, 01 = +1, 11 = -1) becomes (c & 1) << 1 | (c & 2) << 2:
// 0000 = 0, 0010 = +1.0, 1010 = -1.0.
__global__ __launch_bounds__(256) void weights_to_fp4_kernel(const uint32_t* __restrict__ Wp, int64_t n_words,
                                                             int64_t N, int64_t K, uint8_t* __restrict__ W4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_words) return;
    const uint32_t w = Wp[i];
    uint32_t o[2];
#pragma unroll
    for (int half = 0; half < 2; half++) {
        // bit pairs 2*half, 2*half+1 of each byte: weights b + 8*half and b + 4 + 8*half of byte b
        const uint32_t x = (w >> (4 * half)) & 0x0F0F0F0Fu;
        const uint32_t t = (x & 0x03030303u) | ((x & 0x0C0C0C0Cu) << 2);     // byte b: [pair lo | pair hi << 4]
        const uint32_t u = ((t & 0x11111111u) << 1) | ((t & 0x22222222u) << 2);  // each 2-bit code -> FP4 nibble
        // nibble transpose: low nibbles of bytes 0..3, then the high nibbles
        const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
        o[half] = __builtin_amdgcn_perm(hi | (hi >> 4), lo | (lo >> 4), 0x06040200u);
    }
    const int64_t words_per_row = K / 16;
    const int64_t n = i / words_per_row;
    *reinterpret_cast<uint2*>(W4 + fp4_byte_offset(n, 16 * (i - n * words_per_row), N, K)) = make_uint2(o[0], o[1]);
}

}  // namespace

bool gemm_f6f4_eligible(int64_t M, int64_t K, int64_t N) {
    // prefill shapes with at least 128 tiles of 256 x 256 (fewer tiles leave
    // CUs idle; the INT8 path then has smaller tiles); K >= 512 so that the
    // activation kernel writes whole FP6 bytes
    return M > 64 && K >= 512 && K % kBK == 0 && ((M + kF6BM - 1) / kF6BM) * ((N + kF6BN - 1) / kF6BN) >= 128;
}

hipError_t launch_gemm_f6f4(const uint8_t* codes6, const float* xscale, int64_t M, int64_t K, const uint8_t* W4,
                            const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int tiles_n = (int)((N + kF6BN - 1) / kF6BN);
    const int64_t tiles = (int64_t)tiles_n * ((M + kF6BM - 1) / kF6BM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int tt = (int)tiles;
    constexpr int NT = 64 * kF6WGM * kF6WGN;
    // at least 10 waves of tiles over the 256 CUs (one block each): XCDs start 128 x 64 cycles apart
    const int stagger = tt >= 10 * 256 ? 128 : 0;
    if (y_dtype == HBL_F32)
        hipLaunchKernelGGL((gemm_f6f4_kernel<float, kF6BM, kF6BN, kF6WGM, kF6WGN, kF6Stages>), dim3(tt), dim3(NT), 0,
                           s, codes6, xscale, M, K, W4, alpha, N, (float*)Y, tiles_n, tt, stagger);
    else
        hipLaunchKernelGGL((gemm_f6f4_kernel<uint16_t, kF6BM, kF6BN, kF6WGM, kF6WGN, kF6Stages>), dim3(tt), dim3(NT),
                           0, s, codes6, xscale, M, K, W4, alpha, N, (uint16_t*)Y, tiles_n, tt, stagger);
    return hipGetLastError();
}

hipError_t launch_weights_to_fp4(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W4, hipStream_t s) {
    const int64_t n_words = N * K / 16;
    const int64_t blocks = (n_words + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(weights_to_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint32_t*)W_packed,
                       n_words, N, K, W4);
    return hipGetLastError();
}

bool gemm_uses_decode_kernel(int64_t M, int64_t K) {
    return M >= 1 && M <= 64 && !gemv_small_shape(M, K) && K % 256 == 0 && K / 256 <= kDecWaves * kDecMaxSS;
}

hipError_t launch_gemm(const void* codes, const float* xscale, int act_bits, int64_t M, int64_t K,
                       const uint8_t* W_packed, const float* alpha, int64_t N, void* Y, int y_dtype, hipStream_t s,
                       bool dec_tiled) {
    if (M == 0) return hipSuccess;
    const uint8_t* A = (const uint8_t*)codes;
    if (act_bits == 8) {
        return y_dtype == HBL_F32
                   ? launch_typed<8, float>(A, xscale, M, K, W_packed, alpha, N, (float*)Y, s, dec_tiled)
                   : launch_typed<8, uint16_t>(A, xscale, M, K, W_packed, alpha, N, (uint16_t*)Y, s, dec_tiled);
    }
    return y_dtype == HBL_F32
               ? launch_typed<4, float>(A, xscale, M, K, W_packed, alpha, N, (float*)Y, s, dec_tiled)
               : launch_typed<4, uint16_t>(A, xscale, M, K, W_packed, alpha, N, (uint16_t*)Y, s, dec_tiled);
}

}  // namespace hbl
