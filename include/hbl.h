/*
 * hbl.h -- C ABI of libhbl.so, the H-BitLinear forward pass (BitNet v2) on
 * AMD MI355X (gfx950).
 *
 * The layer replaces a standard linear layer y[M][N] = x[M][K] W[N][K]^T
 * (no bias).  Each token row of x is normalised, rotated by an online
 * Hadamard transform, quantised per token to INT8 or INT4, and multiplied
 * against per-tensor absmean-ternarised weights with integer accumulation,
 * then rescaled to float.  Pages followed (their display equations were lost
 * in extraction; the readings are stated per call):
 *   - "新智元: 微软 BitNet v2" repost, section "H-BitLinear模块": the online
 *     Hadamard before activation quantisation, computed by a fast O(n log n)
 *     transform; the per-tensor absmean ternary weight quantiser; the
 *     separate 8-bit and 4-bit activation strategies; the layer formula with
 *     a normalisation LN(.) in front.
 *   - same page, section "BitNet v2：原生4位激活": RMSNorm, no bias, H-BitLinear
 *     only at the attention output Wo and the FFN down projection Wdown; plain
 *     BitLinear (no Hadamard) elsewhere.
 *   - CSDN blog "[论文品鉴] 1-bit LLM", section "量化函数": the threshold form of
 *     the ternariser (inclusive zero band).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major
 *     and contiguous.  The library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is queued on it and the call returns before the GPU finishes.
 *   - Every argument is validated on the host before anything is queued; an
 *     invalid argument returns an error code and queues nothing.  No call
 *     aborts or throws.  HBL_ERR_HIP reports a failed launch; the HIP error
 *     code is then available from hbl_last_hip_error() on the same thread.
 *   - Calls on one stream are ordered; calls that share output or workspace
 *     buffers on different streams race.
 *   - NaN or Inf inputs are outside the contract.
 */
#ifndef HBL_H
#define HBL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HBL_OK = 0,
    HBL_ERR_NULL = 1,        /* a required pointer is NULL */
    HBL_ERR_SHAPE = 2,       /* a size is out of range (M < 0, N or K <= 0, too large) */
    HBL_ERR_NOT_POW2 = 3,    /* hadamard = 1 needs K a power of two */
    HBL_ERR_ALIGN = 4,       /* K % 16 or N % 16 != 0, or a pointer not 16-byte aligned */
    HBL_ERR_DTYPE = 5,       /* unknown hbl_dtype */
    HBL_ERR_BITS = 6,        /* act_bits not 4 or 8, or unknown a4_mode / norm */
    HBL_ERR_WORKSPACE = 7,   /* workspace smaller than the *_workspace_bytes query */
    HBL_ERR_UNSUPPORTED = 8, /* valid request this library does not implement */
    HBL_ERR_HIP = 9          /* a HIP call failed; see hbl_last_hip_error() */
} hbl_status;

typedef enum { HBL_F32 = 0, HBL_BF16 = 1 } hbl_dtype;

typedef enum { HBL_NORM_RMS = 0, HBL_NORM_LN = 1, HBL_NORM_NONE = 2 } hbl_norm;

/* INT4 per-token scale.  The pages announce two different strategies for
 * 8-bit and 4-bit activations but the formulas were lost; the default reads
 * the 4-bit one as absmean with sqrt(7) (beta = mean|z|, codes =
 * clip(rint(z*sqrt7/(beta+eps)), -8, 7), dequant beta/sqrt7), with absmax/7 as
 * the alternative.  sqrt7 is the fp32 constant 0x402953FD. */
typedef enum { HBL_A4_ABSMEAN_SQRT7 = 0, HBL_A4_ABSMAX_7 = 1 } hbl_a4_mode;

typedef struct {
    int32_t act_bits;  /* 8: INT8 absmax codes [M][K] int8; 4: INT4 codes packed [M][K/2] */
    int32_t hadamard;  /* 1: H-BitLinear (online Hadamard), 0: plain BitLinear */
    int32_t norm;      /* hbl_norm; applied before the Hadamard */
    int32_t a4_mode;   /* hbl_a4_mode; ignored when act_bits == 8 */
    float norm_eps;    /* added to the mean square (variance) inside the sqrt */
    float quant_eps;   /* added to the per-token statistic in the quantiser divisor */
} hbl_config;

/* Limits of this library. */
#define HBL_MAX_K 32768
#define HBL_MIN_K 256

/*
 * Weight format (library definition; the pages give none for 2-bit storage).
 *   W_packed: uint8 [N][K/4].  Each ternary value is 2-bit two's complement
 *   (0 -> 00, +1 -> 01, -1 -> 11; 10 never written).  K is cut into aligned
 *   groups of 16; group g of row n owns bytes 4g..4g+3 of that row, and
 *   element k sits in byte 4*(k/16) + k%4 at bits 2*((k%16)/4)..+1.
 *   alpha: one fp32 in device memory, the per-tensor absmean mean|W|.
 * INT8 activation codes: int8 [M][K].  INT4 codes: uint8 [M][K/2], low nibble
 * = even k, high nibble = odd k, 4-bit two's complement.  xscale: fp32 [M],
 * the per-token dequantisation factor (gamma/127, beta/sqrt7 or gamma/7).
 */

/* Bytes of W_packed for an N x K weight (N*K/4).  Errors: NULL, SHAPE, ALIGN. */
hbl_status hbl_packed_weight_bytes(int64_t N, int64_t K, size_t* bytes);

/* Device workspace needed by hbl_quantize_weights (partial sums). */
hbl_status hbl_weight_workspace_bytes(int64_t N, int64_t K, size_t* bytes);

/*
 * Per-tensor absmean ternarisation and packing of latent weights W [N][K]
 * (fp32 or bf16):  alpha = mean|W| over all N*K entries (fp64 sum, rounded
 * to fp32);  W_q = clip(rint(W / (alpha + eps)), -1, 1) with round half to
 * even, so the zero band |W| <= (alpha+eps)/2 is inclusive;  dequant factor
 * is alpha.  Writes W_packed (hbl_packed_weight_bytes) and alpha (1 float,
 * device).  ws must hold hbl_weight_workspace_bytes.  An all-zero W gives
 * alpha = 0 and all-zero codes.  Constraints: N >= 1, K >= 16, K % 16 == 0,
 * N*K < 2^40.
 */
hbl_status hbl_quantize_weights(const void* W, int32_t w_dtype, int64_t N, int64_t K, float eps,
                                uint8_t* W_packed, float* alpha, void* ws, size_t ws_bytes, void* stream);

/* Device workspace needed by hbl_forward and hbl_forward_latent (activation
 * codes + per-token scale; for M <= 64 the codes region is padded to whole
 * 16-row tiles). */
hbl_status hbl_workspace_bytes(int64_t M, int64_t K, const hbl_config* cfg, size_t* bytes);

/*
 * Workspace with which hbl_forward and hbl_forward_latent take their fastest
 * path for an M x K by N x K layer: >= hbl_workspace_bytes(M, K, cfg).  For
 * INT4 activations at prefill sizes (M > 64, K >= 512, at least 128 output
 * tiles of 256 x 256) it adds room for the codes as FP6 and the weights as
 * FP4, and a workspace of this size lets the forward multiply them on the
 * gfx950 FP6 x FP4 matrix cores (twice the INT8 rate).  The products and
 * sums are exact integers there as well, so Y is the same bit for bit with
 * either workspace size (the hardware-format reading of the pages' remark
 * that 4-bit activations suit native low-bit compute, "新智元: 微软 BitNet v2",
 * section "原生4比特盘算").  N in [1, 2^20]; other errors as hbl_workspace_bytes.
 */
hbl_status hbl_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, const hbl_config* cfg, size_t* bytes);

/*
 * Activation half of the layer, per token row m of X [M][K] (fp32 or bf16):
 *   r = norm(x) * gain   (RMS: x/sqrt(mean x^2 + norm_eps); LN: (x-mean)/
 *                          sqrt(var + norm_eps); NONE: x; gain NULL = 1)
 *   z = H_K r             when cfg->hadamard (normalised Sylvester Hadamard,
 *                          natural order, H[i][j] = (-1)^popcount(i&j)/sqrt(K),
 *                          computed by an in-register/LDS fast transform)
 *   s, d from z           INT8: gamma = max|z|, s = 127/(gamma+eps), d = gamma/127
 *                          INT4: see hbl_a4_mode.  A zero statistic gives s = d = 0,
 *                          and so does one whose s overflows fp32 (quant_eps = 0
 *                          and a row below about 1e-37: reading of the lost formula).
 *   q = clip(rint(z*s))   INT8 [-128,127] -> codes int8 [M][K]
 *                          INT4 [-8,7]     -> codes uint8 [M][K/2] (packed)
 *   xscale[m] = d
 * z_debug (nullable): fp32 [M][K] copy of z; s_debug (nullable): fp32 [M]
 * quantiser multiplier s.  Both exist for parity checks.
 * gain (nullable): fp32 [K].
 * Constraints: K a power of two in [256, 32768] (both modes); 0 <= M < 2^31
 * (M == 0 queues nothing); X, codes and z_debug 16-byte aligned.
 */
hbl_status hbl_quantize_activations(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                                    const hbl_config* cfg, void* codes, float* xscale, float* z_debug,
                                    float* s_debug, void* stream);

/*
 * Integer half of the layer: acc[m][n] = sum_k q[m][k] * W_q[n][k] in int32
 * (exact: |acc| <= 128*K < 2^31), then Y[m][n] = fp32(fp32(acc * xscale[m]) *
 * alpha), stored as fp32 or bf16 (round to nearest even).  With xscale = 1 and
 * alpha = 1 the fp32 output equals acc exactly (|acc| < 2^24).  INT8 x ternary
 * products run on the gfx950 i8 matrix cores (MFMA).  Constraints: K in
 * [128, 32768], K % 128 == 0; N in [16, 2^20], N % 16 == 0; 0 <= M <= 2^23 (M == 0
 * queues nothing); codes, W_packed and Y 16-byte aligned.
 */
hbl_status hbl_gemm(const void* codes, const float* xscale, int32_t act_bits, int64_t M, int64_t K,
                    const uint8_t* W_packed, const float* alpha, int64_t N, void* Y, int32_t y_dtype,
                    void* stream);

/*
 * The whole H-BitLinear (or plain BitLinear) forward: hbl_quantize_activations
 * into the workspace, then hbl_gemm.  Y [M][N] fp32 or bf16, bit for bit the
 * result of those two calls.  ws (16-byte aligned) must hold
 * hbl_workspace_bytes(M, K, cfg) (room for the codes followed by xscale); its
 * contents afterwards are unspecified: for one token (M = 1) with K a power
 * of two in [1024, 16384] the whole forward runs as a single launch and the
 * codes never leave the chip; for the other shapes up to 64 tokens that the
 * decode GEMM serves, the codes are kept in a tiled order private to the
 * library.  Constraints: those of both stages.
 */
hbl_status hbl_forward(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                       const uint8_t* W_packed, const float* alpha, int64_t N, const hbl_config* cfg,
                       void* Y, int32_t y_dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole hot path from latent weights, for callers that re-ternarise the
 * weights on every forward (training with latent weights): the results of
 * hbl_quantize_weights(W, w_dtype, N, K, w_eps, W_packed, alpha, wws, ...)
 * followed by hbl_forward(X, ..., W_packed, alpha, ..., Y, ..., ws, ...),
 * bit for bit.  For K <= 2048 it takes three launches instead of four: the
 * activation quantisation and the weight packing share one grid (they do not
 * depend on each other).  W_packed and alpha are outputs (device memory the caller
 * owns, reusable by hbl_forward).  ws must hold hbl_workspace_bytes(M, K,
 * cfg) and wws hbl_weight_workspace_bytes(N, K); contents afterwards are
 * unspecified.  M = 0 only ternarises the weights (X, Y, ws may be NULL).
 * Constraints: those of hbl_quantize_weights and hbl_forward together.
 */
hbl_status hbl_forward_latent(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                              const void* W, int32_t w_dtype, int64_t N, float w_eps, const hbl_config* cfg,
                              uint8_t* W_packed, float* alpha, void* Y, int32_t y_dtype, void* ws,
                              size_t ws_bytes, void* wws, size_t wws_bytes, void* stream);

/*
 * INT4 prefill on the gfx950 FP6 x FP4 matrix cores with the weights held in
 * FP4 (the hardware-format reading of the pages' remark that 4-bit
 * activations suit native low-bit compute for batched inference, "新智元: 微软
 * BitNet v2" repost, section "原生4比特盘算").  Every INT4 code [-8, 7] is exact
 * in FP6 E3M2 and every ternary weight in FP4 E2M1; |acc| <= 8*K <= 2^18, so
 * the fp32 sums are exact integers and Y is the same bit for bit as
 * hbl_forward's with INT4 codes.
 *
 * FP4 weight format (library definition): W4, N*K/2 bytes, each ternary
 * weight one E2M1 nibble: 0 -> 0x0, +1 -> 0x2, -1 -> 0xA.  The order suits
 * the GEMM's loads: rows in bands of 256 (band b: rows 256b .. 256b+R-1, R =
 * min(256, N - 256b)); in a band, K step s (weights 128s .. 128s+127, 64
 * bytes per row) of all R rows is one block of R*64 bytes at byte
 * 256b*K/2 + 64*s*R, row r of the band at +64r; inside those 64 bytes the
 * 16 bytes of weights 32c .. 32c+31 sit at +16*(c ^ ((r >> 2) & 3)), weight k
 * at nibble k % 32 (low nibble first).  hbl_fp4_weight_bytes: N*K/2
 * (constraints as hbl_packed_weight_bytes, and K % 128 == 0, else
 * HBL_ERR_ALIGN).  hbl_pack_fp4: W_packed (the 2-bit layout of
 * hbl_quantize_weights) -> W4, the same ternary values; a deployment converts
 * once per weight.  Both buffers 16-byte aligned.
 *
 * FP6 codes: M*K*3/4 bytes (hbl_fp6_codes_bytes), the INT4 codes of
 * hbl_quantize_activations as E3M2 fields in the operand order of the
 * FP6 x FP4 GEMM (blocks of one K step of 256 rows); the order is private to
 * this library, made for M and K together, and read only by hbl_gemm_fp6fp4
 * with the same M and K.  hbl_quantize_activations_fp6 writes them (same
 * computation and xscale as hbl_quantize_activations with cfg->act_bits = 4,
 * which it requires; K a power of two in [512, 32768]).
 * hbl_gemm_fp6fp4: Y = fp32(fp32(acc * xscale[m]) * alpha), fp32 or bf16, from
 * FP6 codes and FP4 weights; K in [512, 32768], K % 128 == 0, N in [16, 2^20],
 * N % 16 == 0, 0 <= M <= 2^23 (M == 0 queues nothing).
 * hbl_forward_fp4: hbl_quantize_activations_fp6 into the workspace
 * (hbl_forward_fp4_workspace_bytes: the FP6 codes, then xscale, each region
 * 256-byte aligned), then hbl_gemm_fp6fp4; bit for bit hbl_forward with the
 * same config on the same ternary values.  Constraints: those of both.
 */
hbl_status hbl_fp4_weight_bytes(int64_t N, int64_t K, size_t* bytes);
hbl_status hbl_pack_fp4(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W4, void* stream);
hbl_status hbl_fp6_codes_bytes(int64_t M, int64_t K, size_t* bytes);
hbl_status hbl_quantize_activations_fp6(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                                        const hbl_config* cfg, uint8_t* codes6, float* xscale, void* stream);
hbl_status hbl_gemm_fp6fp4(const uint8_t* codes6, const float* xscale, int64_t M, int64_t K, const uint8_t* W4,
                           const float* alpha, int64_t N, void* Y, int32_t y_dtype, void* stream);
hbl_status hbl_forward_fp4_workspace_bytes(int64_t M, int64_t K, const hbl_config* cfg, size_t* bytes);
hbl_status hbl_forward_fp4(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                           const uint8_t* W4, const float* alpha, int64_t N, const hbl_config* cfg, void* Y,
                           int32_t y_dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * Low-bit attention states, beside the layer ("新智元: 微软 BitNet v2" repost,
 * section "实验结果": after RoPE the Q, K and V heads are quantised directly to
 * unsigned integers by absmax, with no calibration; a 3-bit KV cache keeps
 * the accuracy of a full-precision one).  For every token m and head h of
 * X [M][H][D] (fp32 or bf16; post-RoPE states; row-major, so also [M][H*D]):
 *   gamma = max_d |x|, Qp = 2^(bits-1) - 1, s = Qp/(gamma + eps) (fp32),
 *   d = gamma/Qp,  u = clamp(rint(x*s), -Qp, Qp) + 2^(bits-1)  in [1, 2^bits - 1]
 *   (round half to even; gamma == 0 gives d = 0 and every u = 2^(bits-1), as
 *   does a gamma so small that s overflows fp32 when eps = 0;
 *   dequantised value (u - 2^(bits-1)) * d).  The formula is the reading of
 *   the page taken here: a symmetric absmax quantiser stored with an offset.
 * codes: uint8 [M][H][D*bits/8]: bits = 8 one byte per code; 4 two per byte,
 * even d in the low nibble; 3 code d at bits 3d..3d+2 of the head vector's
 * little-endian bit string.  scales: fp32 [M][H] = d.  All device memory.
 * Constraints: bits in {3, 4, 8}; D in {32, 64, 128, 256}; H >= 1; M >= 0
 * (M == 0 queues nothing); M*H*D < 2^40; eps >= 0; X and codes 16-byte
 * aligned, scales 4-byte aligned.
 */
hbl_status hbl_quantize_heads(const void* X, int32_t x_dtype, int64_t M, int64_t H, int64_t D, int32_t bits,
                              float eps, uint8_t* codes, float* scales, void* stream);

/*
 * The layer's backward with the straight-through estimator (training through
 * the low-bit quantisers with it: the xdnf.cn page on BitNet v2, section
 * "研究方法"; training with low-bit activations and ternary weights: the
 * "新智元: 微软 BitNet v2" repost, section "BitNet v2：原生4位激活").  The quantisers are identities in the
 * backward, so for the forward y = alpha * d * (q . Wq^T) of hbl_forward:
 *   dZ = alpha * dY . Wq                 [M][K]
 *   dR = H dZ (normalised Sylvester, symmetric; dR = dZ when cfg->hadamard = 0)
 *   dX = norm'(x)^T dR: RMS c g dR - (c^3/K) x sum(g dR x); LN
 *        c (a - mean(a) - xh mean(a xh)) with a = g dR, xh = (x - mu) c;
 *        none g dR  (c = 1/sqrt(mean + norm_eps) as in the forward)
 *   dW = dY^T . (d * q)                  [N][K], q and d the forward's codes
 *        and factors (computed again from X)
 * dY [M][N] and X [M][K] fp32 or bf16; gain fp32 [K] or NULL; W_packed and
 * alpha as for hbl_forward.  dX fp32 [M][K]; dW fp32 [N][K] or NULL (then
 * only dX).  The two products run on the bf16 matrix cores with fp32 sums; dY
 * (and dY * d) are split into a bf16 high part and a bf16 remainder, so the
 * result agrees with the exact one to about 1e-5 of the row's largest value.
 * ws (16-byte aligned) must hold hbl_backward_workspace_bytes(M, K, N, cfg,
 * dW != NULL).  Constraints: those of hbl_forward, K >= 512, M and N <= 2^21;
 * dY, X, dX, dW 16-byte aligned, gain 4-byte aligned.
 */
hbl_status hbl_backward_workspace_bytes(int64_t M, int64_t K, int64_t N, const hbl_config* cfg, int32_t with_dw,
                                        size_t* bytes);
hbl_status hbl_backward(const void* dY, int32_t dy_dtype, const void* X, int32_t x_dtype, int64_t M, int64_t K,
                        const float* gain, const uint8_t* W_packed, const float* alpha, int64_t N,
                        const hbl_config* cfg, float* dX, float* dW, void* ws, size_t ws_bytes, void* stream);

/*
 * Base-3 weight storage for the weight-bandwidth-bound decode regime (the
 * CSDN post "[论文品鉴] 1-bit LLM", section "掩码存储": several ternary weights
 * packed into one integer, five per 8-bit byte).  Layout W3 uint8 [N][RB],
 * RB = 16 * ceil(K / 80): byte j of row n holds the weights k = 5j .. 5j+4 as
 * base-3 digits, byte = sum_{i<5} (W_q[n][5j+i] + 1) * 3^i (first weight least
 * significant; weights past K count as 0), 1.6 bits per weight.  The digit
 * order and the row padding are the reading taken here; the page fixes only
 * five weights per byte.
 * hbl_base3_weight_bytes: N * RB.  Constraints as hbl_packed_weight_bytes.
 * hbl_pack_base3: W_packed (the 2-bit layout of hbl_quantize_weights) -> W3,
 * the same ternary values.  Both device buffers 16-byte aligned.
 */
hbl_status hbl_base3_weight_bytes(int64_t N, int64_t K, size_t* bytes);
hbl_status hbl_pack_base3(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W3, void* stream);

/*
 * hbl_gemm with base-3 weights, for 1 to 4 tokens: Y = rescale(sum_k q W_q),
 * bit for bit the output of hbl_gemm on the same ternary values (int32 sums
 * on the vector ALU's dot-product instructions, then y = fp32(fp32(acc *
 * xscale[m]) * alpha)).  codes as for hbl_gemm (row-major).  Constraints:
 * 0 <= M <= 4 (M == 0 queues nothing); K % 16 == 0, 16 <= K <= 16384;
 * 1 <= N <= 2^20; codes, W3 and Y 16-byte aligned.
 */
hbl_status hbl_gemm_base3(const void* codes, const float* xscale, int32_t act_bits, int64_t M, int64_t K,
                          const uint8_t* W3, const float* alpha, int64_t N, void* Y, int32_t y_dtype, void* stream);

/*
 * hbl_forward with base-3 weights for 1 to 4 tokens: hbl_quantize_activations
 * into the workspace (hbl_workspace_bytes), then hbl_gemm_base3.  Bit for bit
 * hbl_forward on the same ternary values.  Constraints: those of
 * hbl_quantize_activations and hbl_gemm_base3 together (K a power of two in
 * [256, 16384], M <= 4).
 */
hbl_status hbl_forward_base3(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                             const uint8_t* W3, const float* alpha, int64_t N, const hbl_config* cfg, void* Y,
                             int32_t y_dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * hbl_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and result, bit for bit, with the workspace taken from a
 * static device array of HBL_NOALLOC_SCRATCH_BYTES inside the library (each
 * GPU it runs on holds one until the process ends).  The caller still passes
 * X, the weights, alpha and Y.  Returns HBL_ERR_WORKSPACE when the shape's
 * hbl_workspace_bytes(M, K, cfg) exceeds HBL_NOALLOC_SCRATCH_BYTES; otherwise
 * the errors and constraints of hbl_forward.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, or unordered host threads) race.
 */
#define HBL_NOALLOC_SCRATCH_BYTES (32u << 20)
hbl_status hbl_forward_noalloc(const void* X, int32_t x_dtype, int64_t M, int64_t K, const float* gain,
                               const uint8_t* W_packed, const float* alpha, int64_t N, const hbl_config* cfg,
                               void* Y, int32_t y_dtype, void* stream);

/* Static description of a status code (never NULL). */
const char* hbl_status_string(hbl_status status);

/* The hipError_t of the last HBL_ERR_HIP returned on this thread (0 if none). */
int32_t hbl_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HBL_H */
