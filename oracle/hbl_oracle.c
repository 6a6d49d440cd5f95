/*
 * hbl_oracle.c -- plain, slow, obviously-correct CPU oracle for the H-BitLinear
 * forward pass (BitNet v2).  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg may call it; the product path
 * (the HIP library) never does, and shares no code, header or table with it.
 *
 * Sources (web pages about BitNet v2; their display equations were lost in
 * extraction, so each step below states which passage it follows and, where
 * the page is silent, which reading it takes):
 *   [XZY]  "新智元: 微软 BitNet v2" repost (0755model.com), sections
 *          "BitNet v2：原生4位激活" and "H-BitLinear模块"
 *   [CSDN] "[论文品鉴] 1-bit LLM" (blog.csdn.net), sections "掩码存储" and "量化函数"
 *   [XDNF] "【AI论文】BitNet v2：针对1位LLM的原生4位激活和哈达玛变换" (xdnf.cn)
 *   [SXAI] "AI极简主义革命：BitNet v2如何用4位激活重塑大模型部署与能效", §2.3.2
 *
 * Every function is a direct statement of a definition:
 *   O1  alpha   = mean |W| over the whole tensor            (per-tensor absmean, [XZY] H-BitLinear)
 *   O2  W_q     = clamp(rint(W / (alpha+eps)), -1, 1)          (ternary; zero band |w| <= alpha/2, [CSDN] 量化函数)
 *   O3  pack    2-bit two's complement, 4 per byte; in each aligned group of
 *               16 k, byte (k%4) holds field ((k%16)/4)  (the library's format)
 *   O4  x       = fp32(X)  (bf16 -> fp32 is exact)
 *   O5  r       = RMSNorm / LayerNorm / identity of x, in fp64  ([XZY] layer formula uses LN; architecture uses RMSNorm)
 *   O6  z       = H_K r, H_K[i][j] = (-1)^popcount(i&j) / sqrt(K)  (normalised Sylvester, dense, fp64)
 *   O7  scale   INT8: gamma = max|z|, s = 127/(gamma+eps), d = gamma/127
 *               INT4: beta = mean|z|, s = sqrt7/(beta+eps), d = beta/sqrt7 (default)
 *                     or gamma = max|z|, s = 7/(gamma+eps), d = gamma/7     (alternative)
 *   O8  q       = clamp(rint(fp32(z*s)), lo, hi)   INT8 [-128,127], INT4 [-8,7]; INT4 packs 2/byte
 *   O9  acc     = sum_k q[m][k] * W_q[n][k]   (int64 triple loop, stored as int32)
 *   O10 y       = fp32(fp32(acc * d[m]) * alpha)
 *   O11 beside the layer: low-bit attention states, per (token, head) absmax
 *               to unsigned b-bit integers (b = 3, 4, 8)   ([XZY] 实验结果)
 *   O12 the layer's straight-through backward: dX through H and the norm, dW
 *   O13 base-3 weight storage: five ternary weights per byte   ([CSDN] 掩码存储)
 *   O14 FP4 weight storage: one ternary weight per 4-bit E2M1 code (the
 *       format of the FP6 x FP4 prefill path; [XZY] 原生4比特盘算)
 *
 * Rounding is round-half-to-even (rint under the default FP environment)
 * everywhere.  No step is fused, blocked or reordered beyond these definitions.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared hbl_oracle.c -o libhbl_oracle.so -lm
 * (no -ffast-math, no contraction: every fp32 operation rounds exactly as written.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HBO_OK 0
#define HBO_ERR 1

/* fp32 nearest to sqrt(7) (2.6457512...), bit pattern 0x402953FD.  Used by the
 * INT4 absmean quantiser; stated as a bit pattern so that no library sqrt
 * rounding enters the definition. */
static float hbo_sqrt7_f32(void) {
    union { uint32_t u; float f; } v;
    v.u = 0x402953FDu;
    return v.f;
}

int hbo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void hbo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- O4 ---- */
/* bf16 -> fp32: the bf16 bit pattern is the top half of the fp32 pattern. */
void hbo_bf16_to_f32(const uint16_t* x, int64_t n, float* out) {
    for (int64_t i = 0; i < n; i++) {
        union { uint32_t u; float f; } v;
        v.u = ((uint32_t)x[i]) << 16;
        out[i] = v.f;
    }
}

/* fp32 -> bf16, round to nearest even (used only for a bf16 output variant). */
void hbo_f32_to_bf16(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) {
        union { uint32_t u; float f; } v;
        v.f = x[i];
        uint32_t lsb = (v.u >> 16) & 1u;
        out[i] = (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
    }
}

/* ---------------------------------------------------------- O1, O2 ------ */
/* alpha = (sum |W| in fp64, sequential) / count, rounded to fp32.
 * Per-tensor absmean [XZY, H-BitLinear module]. */
float hbo_weight_alpha(const float* W, int64_t count) {
    double s = 0.0;
    for (int64_t i = 0; i < count; i++) s += fabs((double)W[i]);
    if (count <= 0) return 0.0f;
    return (float)(s / (double)count);
}

/* Ternarise one tensor of `count` latent weights with the given alpha.
 * t = fp32(W / fp32(alpha + eps)); W_q = clamp(rint(t), -1, 1).
 * With round-half-even, |t| = 0.5 maps to 0, so the zero band -D <= w <= D of
 * the threshold form ([CSDN] 量化函数) is inclusive with D = (alpha+eps)/2.
 * alpha + eps == 0 (an all-zero tensor with eps = 0) gives all zeros. */
void hbo_ternarize(const float* W, int64_t count, float alpha, float eps, int8_t* Wq) {
    float den = alpha + eps;
    for (int64_t i = 0; i < count; i++) {
        if (den == 0.0f) { Wq[i] = 0; continue; }
        float t = W[i] / den;
        float r = rintf(t);
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        Wq[i] = (int8_t)r;
    }
}

/* ---------------------------------------------------------------- O3 ---- */
/* 2-bit packing of a [N][K] ternary matrix into bytes [N][K/4].  The pages
 * give no 2-bit layout (they describe 5-trits-per-byte and bitmask+sign
 * storage, [CSDN] 掩码存储), so this one is the library's own definition:
 *   code:     2-bit two's complement, 0 -> 00, +1 -> 01, -1 -> 11 (10 unused)
 *   position: K is cut into aligned groups of 16; the group g of row n owns
 *             bytes 4g..4g+3 of that row; element k goes to byte 4*(k/16) + k%4,
 *             bits 2*((k%16)/4) and 2*((k%16)/4)+1.
 * So byte b of a group holds the four elements whose index is b mod 4, in
 * increasing k from the lowest bit pair.  Requires K % 16 == 0. */
static int64_t hbo_tern_byte(int64_t k) { return 4 * (k / 16) + (k % 4); }
static int hbo_tern_shift(int64_t k) { return (int)(2 * ((k % 16) / 4)); }

int hbo_pack_ternary(const int8_t* Wq, int64_t N, int64_t K, uint8_t* Wp) {
    if (K % 16) return HBO_ERR;
    memset(Wp, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int v = Wq[n * K + k];
            uint8_t code = (v == 0) ? 0u : (v == 1 ? 1u : 3u);
            Wp[n * (K / 4) + hbo_tern_byte(k)] |= (uint8_t)(code << hbo_tern_shift(k));
        }
    return HBO_OK;
}

/* Inverse of hbo_pack_ternary; the unused code 10 decodes to 2 so that a
 * corrupted byte is visible. */
int hbo_unpack_ternary(const uint8_t* Wp, int64_t N, int64_t K, int8_t* Wq) {
    if (K % 16) return HBO_ERR;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            int code = (Wp[n * (K / 4) + hbo_tern_byte(k)] >> hbo_tern_shift(k)) & 3;
            Wq[n * K + k] = (int8_t)(code == 0 ? 0 : (code == 1 ? 1 : (code == 3 ? -1 : 2)));
        }
    return HBO_OK;
}

/* O1-O3 in one call: alpha from the whole tensor, then ternarise and pack. */
int hbo_quantize_weights(const float* W, int64_t N, int64_t K, float eps,
                         int8_t* Wq, uint8_t* Wp, float* alpha_out) {
    if (N <= 0 || K <= 0 || K % 16) return HBO_ERR;
    float alpha = hbo_weight_alpha(W, N * K);
    hbo_ternarize(W, N * K, alpha, eps, Wq);
    *alpha_out = alpha;
    return hbo_pack_ternary(Wq, N, K, Wp);
}

/* ---------------------------------------------------------------- O5 ---- */
/* norm: 0 = RMSNorm, 1 = LayerNorm, 2 = none.  fp64 throughout.
 * RMS:  r_k = x_k / sqrt(sum x^2 / K + eps) * g_k
 * LN:   r_k = (x_k - mu) / sqrt(sum (x - mu)^2 / K + eps) * g_k
 * gain == NULL means g = 1.  There is no bias ([XZY] "BitNet v2：原生4位激活"). */
void hbo_norm_row(const float* x, int64_t K, const float* gain, int norm, float eps, double* r) {
    if (norm == 2) {
        for (int64_t k = 0; k < K; k++) r[k] = (double)x[k] * (gain ? (double)gain[k] : 1.0);
        return;
    }
    double mu = 0.0;
    if (norm == 1) {
        for (int64_t k = 0; k < K; k++) mu += (double)x[k];
        mu /= (double)K;
    }
    double ss = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double c = (double)x[k] - mu;
        ss += c * c;
    }
    double den = sqrt(ss / (double)K + (double)eps);
    for (int64_t k = 0; k < K; k++) {
        double v = ((double)x[k] - mu) / den;
        r[k] = v * (gain ? (double)gain[k] : 1.0);
    }
}

/* ---------------------------------------------------------------- O6 ---- */
/* Dense normalised Sylvester Hadamard, natural order:
 * z_i = sum_j (-1)^popcount(i & j) r_j / sqrt(K), K a power of two.
 * The +-1 entries and orthogonal rows are the properties the pages state
 * ([XZY] H-BitLinear module, Hadamard paragraph); the O(K log K) fast
 * transform the pages mention computes this same product, which is why the
 * oracle keeps the dense O(K^2) form.  The matrix is never materialised. */
void hbo_hadamard_row(const double* r, int64_t K, double* z) {
    double inv = 1.0 / sqrt((double)K);
    for (int64_t i = 0; i < K; i++) {
        double acc = 0.0;
        for (int64_t j = 0; j < K; j++) {
            int odd = __builtin_popcountll((unsigned long long)(i & j)) & 1;
            acc += (odd ? -1.0 : 1.0) * r[j];
        }
        z[i] = acc * inv;
    }
}

/* ------------------------------------------------------------ O7, O8 ---- */
/* Per-token activation scale.  bits = 8: absmax.  bits = 4: a4_mode 0 =
 * absmean with sqrt7, a4_mode 1 = absmax with 7.  Outputs the quantiser
 * multiplier s and the dequantisation factor d.  A zero statistic gives
 * s = d = 0 (all codes 0). */
int hbo_act_scale(const float* z, int64_t K, int bits, int a4_mode, float eps, float* s_out, float* d_out) {
    float stat, num;
    if (bits == 8 || (bits == 4 && a4_mode == 1)) {
        float g = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float a = fabsf(z[k]);
            if (a > g) g = a;
        }
        stat = g;
        num = (bits == 8) ? 127.0f : 7.0f;
    } else if (bits == 4 && a4_mode == 0) {
        double s = 0.0;
        for (int64_t k = 0; k < K; k++) s += fabs((double)z[k]);
        stat = (float)(s / (double)K);
        num = hbo_sqrt7_f32();
    } else {
        return HBO_ERR;
    }
    if (stat == 0.0f) { *s_out = 0.0f; *d_out = 0.0f; return HBO_OK; }
    float den = stat + eps;
    float s = num / den;
    /* With eps = 0 a statistic below num / FLT_MAX (about 3.7e-37 for INT8)
     * makes the multiplier overflow to +inf, and 0 * inf has no code.  The
     * pages never reach this range; the reading taken: such a row is
     * treated as a zero statistic (s = d = 0, all codes 0). */
    if (isinf(s)) { *s_out = 0.0f; *d_out = 0.0f; return HBO_OK; }
    *s_out = s;
    *d_out = stat / num;
    return HBO_OK;
}

/* q_k = clamp(rint(fp32(z_k * s)), lo, hi): one fp32 multiply, then
 * round-half-even, then clip to the signed range of the bit width. */
int hbo_act_codes(const float* z, int64_t K, int bits, float s, int8_t* q) {
    float lo, hi;
    if (bits == 8) { lo = -128.0f; hi = 127.0f; }
    else if (bits == 4) { lo = -8.0f; hi = 7.0f; }
    else return HBO_ERR;
    for (int64_t k = 0; k < K; k++) {
        float t = z[k] * s;   /* a single rounded fp32 product */
        float r = rintf(t);
        if (r > hi) r = hi;
        if (r < lo) r = lo;
        q[k] = (int8_t)r;
    }
    return HBO_OK;
}

/* INT4 packing of [M][K] codes into bytes [M][K/2]: low nibble = even k,
 * high nibble = odd k, each 4-bit two's complement.  Requires K % 2 == 0. */
int hbo_pack_int4(const int8_t* q, int64_t M, int64_t K, uint8_t* p) {
    if (K % 2) return HBO_ERR;
    for (int64_t m = 0; m < M; m++)
        for (int64_t k2 = 0; k2 < K / 2; k2++) {
            uint8_t lo = (uint8_t)(q[m * K + 2 * k2] & 0xF);
            uint8_t hi = (uint8_t)(q[m * K + 2 * k2 + 1] & 0xF);
            p[m * (K / 2) + k2] = (uint8_t)(lo | (hi << 4));
        }
    return HBO_OK;
}

int hbo_unpack_int4(const uint8_t* p, int64_t M, int64_t K, int8_t* q) {
    if (K % 2) return HBO_ERR;
    for (int64_t m = 0; m < M; m++)
        for (int64_t k = 0; k < K; k++) {
            int nib = (p[m * (K / 2) + k / 2] >> (4 * (k % 2))) & 0xF;
            q[m * K + k] = (int8_t)(nib >= 8 ? nib - 16 : nib);
        }
    return HBO_OK;
}

/* O4-O8 for a batch of rows.  X is fp32 [M][K] (bf16 callers convert with
 * hbo_bf16_to_f32 first, which is exact).  hadamard = 1: H-BitLinear,
 * hadamard = 0: plain BitLinear (same steps without O6).
 * Outputs (all caller-allocated, host memory):
 *   z_out [M][K] fp32 (nullable), q [M][K] int8 codes, s_out/d_out [M].
 * Rows are independent; OpenMP splits them over threads. */
int hbo_quantize_activations(const float* X, int64_t M, int64_t K, const float* gain,
                             int norm, float norm_eps, int hadamard, int bits, int a4_mode,
                             float quant_eps, float* z_out, int8_t* q, float* s_out, float* d_out) {
    if (M < 0 || K <= 0) return HBO_ERR;
    if (hadamard && (K & (K - 1))) return HBO_ERR;
    if (!(bits == 8 || bits == 4)) return HBO_ERR;
    int err = 0;
#pragma omp parallel
    {
        double* r = (double*)malloc(sizeof(double) * (size_t)K);
        double* zd = (double*)malloc(sizeof(double) * (size_t)K);
        float* zf = (float*)malloc(sizeof(float) * (size_t)K);
        if (!r || !zd || !zf) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t m = 0; m < M; m++) {
                hbo_norm_row(X + m * K, K, gain, norm, norm_eps, r);
                if (hadamard) {
                    hbo_hadamard_row(r, K, zd);
                    for (int64_t k = 0; k < K; k++) zf[k] = (float)zd[k];
                } else {
                    for (int64_t k = 0; k < K; k++) zf[k] = (float)r[k];
                }
                if (z_out) memcpy(z_out + m * K, zf, sizeof(float) * (size_t)K);
                hbo_act_scale(zf, K, bits, a4_mode, quant_eps, &s_out[m], &d_out[m]);
                hbo_act_codes(zf, K, bits, s_out[m], q + m * K);
            }
        }
        free(r); free(zd); free(zf);
    }
    return err ? HBO_ERR : HBO_OK;
}

/* ---------------------------------------------------------------- O9 ---- */
/* acc[m][n] = sum_k q[m][k] * Wq[n][k], int64 accumulation, stored as int32.
 * Returns HBO_ERR if any |acc| >= 2^31 (cannot happen for K <= 2^16 with
 * INT8 codes and ternary weights). */
int hbo_int_gemm(const int8_t* q, const int8_t* Wq, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; k++) s += (int64_t)q[m * K + k] * (int64_t)Wq[n * K + k];
            if (s >= 2147483648LL || s < -2147483648LL) {
#pragma omp atomic write
                err = 1;
            }
            acc[m * N + n] = (int32_t)s;
        }
    return err ? HBO_ERR : HBO_OK;
}

/* --------------------------------------------------------------- O10 ---- */
/* y[m][n] = fp32(fp32(float(acc) * d[m]) * alpha): two rounded fp32 products,
 * no bias. */
void hbo_rescale(const int32_t* acc, const float* d, float alpha, int64_t M, int64_t N, float* y) {
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            float t = (float)acc[m * N + n] * d[m];
            y[m * N + n] = t * alpha;
        }
}

/* O4-O10: the whole forward for M rows of fp32 input and a ternary weight
 * matrix already quantised (Wq [N][K] int8, alpha).  Per-row intermediates
 * are returned when the pointers are non-NULL. */
int hbo_forward(const float* X, int64_t M, int64_t K, const float* gain, int norm, float norm_eps,
                int hadamard, int bits, int a4_mode, float quant_eps,
                const int8_t* Wq, float alpha, int64_t N,
                float* y, int32_t* acc_out, int8_t* q_out, float* d_out, float* z_out) {
    if (M < 0 || N <= 0 || K <= 0) return HBO_ERR;
    int8_t* q = q_out ? q_out : (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
    float* s = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    float* d = d_out ? d_out : (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int32_t* acc = acc_out ? acc_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * N > 0 ? M * N : 1));
    int rc = HBO_ERR;
    if (q && s && d && acc) {
        rc = hbo_quantize_activations(X, M, K, gain, norm, norm_eps, hadamard, bits, a4_mode,
                                      quant_eps, z_out, q, s, d);
        if (rc == HBO_OK) rc = hbo_int_gemm(q, Wq, M, N, K, acc);
        if (rc == HBO_OK) hbo_rescale(acc, d, alpha, M, N, y);
    }
    if (!q_out) free(q);
    free(s);
    if (!d_out) free(d);
    if (!acc_out) free(acc);
    return rc;
}

/* --------------------------------------------------------------- O11 ---- */
/* Low-bit attention states, the step beside the layer in [XZY] "实验结果"
 * (low-bit attention, tables 2 and 3): after RoPE the Q, K and V states of
 * every head are quantised directly to unsigned integers by absmax, with no
 * calibration data, and a 3-bit KV cache keeps the accuracy of a full one.
 * The formula is not on the pages; the reading taken: a symmetric absmax
 * quantiser per (token, head) whose signed codes are stored with the offset
 * 2^(b-1), so every code is an unsigned b-bit integer:
 *   gamma = max_d |x[d]|  (x = fp32 values of one head vector, D of them)
 *   Qp = 2^(b-1) - 1;  s = fp32(Qp / fp32(gamma + eps));  d = fp32(gamma / Qp)
 *   u[d] = clamp(rint(fp32(x[d] * s)), -Qp, Qp) + 2^(b-1)      in [1, 2^b - 1]
 *   gamma == 0: s = 0, d = 0, every u = 2^(b-1).   Dequantised: (u - 2^(b-1)) * d.
 * Packing of one head vector (D codes): b = 8 one byte per code; b = 4 two per
 * byte, even index in the low nibble; b = 3 code j in bits 3j .. 3j+2 of the
 * vector's little-endian bit string (8 codes per 3 bytes).
 * X [M][H][D] fp32, codes [M][H][D*b/8], d_out [M][H]. */
int hbo_quantize_heads(const float* X, int64_t M, int64_t H, int64_t D, int bits, float eps, uint8_t* codes,
                       float* d_out) {
    if (M < 0 || H < 1 || D < 8 || D % 8 != 0 || (bits != 3 && bits != 4 && bits != 8)) return HBO_ERR;
    const int zp = 1 << (bits - 1), qp = zp - 1;
    const int64_t vb = D * bits / 8;  /* bytes per packed head vector */
    for (int64_t v = 0; v < M * H; v++) {
        const float* x = X + v * D;
        float gamma = 0.f;
        for (int64_t j = 0; j < D; j++) {
            const float a = fabsf(x[j]);
            if (a > gamma) gamma = a;
        }
        const float den = gamma + eps;
        const float s = gamma == 0.f ? 0.f : (float)qp / den;
        d_out[v] = gamma == 0.f ? 0.f : gamma / (float)qp;
        if (isinf(s)) {
            /* eps = 0 and gamma below qp / FLT_MAX: the multiplier overflows;
             * the vector is treated as gamma == 0 (the reading of O7). */
            d_out[v] = 0.f;
            memset(codes + v * vb, 0, (size_t)vb);
            for (int64_t j = 0; j < D; j++) {
                if (bits == 8) codes[v * vb + j] = (uint8_t)zp;
                else if (bits == 4) codes[v * vb + j / 2] |= (uint8_t)(zp << (4 * (j % 2)));
                else codes[v * vb + (3 * j + 2) / 8] |= (uint8_t)(1u << ((3 * j + 2) % 8));
            }
            continue;
        }
        uint8_t* out = codes + v * vb;
        memset(out, 0, (size_t)vb);
        for (int64_t j = 0; j < D; j++) {
            float t = x[j] * s;
            if (t < (float)-qp) t = (float)-qp;
            if (t > (float)qp) t = (float)qp;
            const int u = (int)rintf(t) + zp;
            if (bits == 8) {
                out[j] = (uint8_t)u;
            } else if (bits == 4) {
                out[j / 2] |= (uint8_t)(u << (4 * (j % 2)));
            } else {
                for (int b = 0; b < 3; b++)
                    if ((u >> b) & 1) out[(3 * j + b) / 8] |= (uint8_t)(1u << ((3 * j + b) % 8));
            }
        }
    }
    return HBO_OK;
}

/* The inverse of O11's packing: D codes per head vector back to one byte each. */
int hbo_unpack_heads(const uint8_t* codes, int64_t V, int64_t D, int bits, uint8_t* u) {
    if (V < 0 || D < 8 || D % 8 != 0 || (bits != 3 && bits != 4 && bits != 8)) return HBO_ERR;
    const int64_t vb = D * bits / 8;
    for (int64_t v = 0; v < V; v++)
        for (int64_t j = 0; j < D; j++) {
            const uint8_t* in = codes + v * vb;
            int c = 0;
            if (bits == 8) c = in[j];
            else if (bits == 4) c = (in[j / 2] >> (4 * (j % 2))) & 15;
            else
                for (int b = 0; b < 3; b++) c |= ((in[(3 * j + b) / 8] >> ((3 * j + b) % 8)) & 1) << b;
            u[v * D + j] = (uint8_t)c;
        }
    return HBO_OK;
}

/* --------------------------------------------------------------- O12 ---- */
/* The layer's backward with the straight-through estimator, the training
 * step beside the forward ([XZY] "BitNet v2：原生4位激活": the model is trained
 * with low-bit activations and ternary weights; the quantisers are passed
 * straight through).  With y[m][n] = alpha * d[m] * sum_k q[m][k] Wq[n][k] and
 * the quantisers taken as identities in the backward (d*q stands for z, and
 * alpha*Wq for the latent W):
 *   dz[m][k] = alpha * sum_n dY[m][n] * Wq[n][k]
 *   dr       = H dz  (H is the symmetric orthonormal Sylvester matrix; = dz
 *              for plain BitLinear)
 *   dx       = the transpose of the norm's Jacobian applied to dr, for
 *              r = norm(x) * g (O5):
 *     RMS:  c = 1/sqrt(sum x^2 / K + eps):
 *           dx_j = c g_j dr_j - (c^3 / K) x_j sum_k g_k dr_k x_k
 *     LN:   c = 1/sqrt(sum (x - mu)^2 / K + eps), xh = (x - mu) c, a = g dr:
 *           dx_j = c (a_j - mean(a) - xh_j mean(a xh))
 *     none: dx_j = g_j dr_j
 *   dW[n][k] = sum_m dY[m][n] * d[m] * q[m][k]   (q, d of the forward, O4-O8)
 * All in fp64.  dX [M][K] and dW [N][K] (nullable) are fp64 outputs. */
/* O12, weight part: dW[n][k] = sum_m dY[m][n] * d[m] * q[m][k] for given codes
 * q [M][K] and dequantisation factors d [M] (fp64). */
void hbo_weight_grad(const float* dY, const int8_t* q, const float* d, int64_t M, int64_t N, int64_t K, double* dW) {
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; m++) acc += (double)dY[m * N + n] * (double)d[m] * (double)q[m * K + k];
            dW[n * K + k] = acc;
        }
}

int hbo_backward(const float* dY, const float* X, int64_t M, int64_t K, const float* gain, int norm, float norm_eps,
                 int hadamard, int bits, int a4_mode, float quant_eps, const int8_t* Wq, float alpha, int64_t N,
                 double* dX, double* dW) {
    if (M < 0 || K <= 0 || N <= 0) return HBO_ERR;
    if (hadamard && (K & (K - 1))) return HBO_ERR;
    double* dz = (double*)malloc(sizeof(double) * (size_t)K);
    double* dr = (double*)malloc(sizeof(double) * (size_t)K);
    int8_t* q = (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
    float* s = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    float* d = (float*)malloc(sizeof(float) * (size_t)(M > 0 ? M : 1));
    int rc = HBO_ERR;
    if (dz && dr && q && s && d) {
        rc = HBO_OK;
        for (int64_t m = 0; m < M; m++) {
            const float* x = X + m * K;
            for (int64_t k = 0; k < K; k++) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; n++) acc += (double)dY[m * N + n] * (double)Wq[n * K + k];
                dz[k] = (double)alpha * acc;
            }
            if (hadamard) hbo_hadamard_row(dz, K, dr);
            else memcpy(dr, dz, sizeof(double) * (size_t)K);
            double* out = dX + m * K;
            if (norm == 2) {
                for (int64_t k = 0; k < K; k++) out[k] = (gain ? (double)gain[k] : 1.0) * dr[k];
            } else if (norm == 0) {
                double ss = 0.0, t = 0.0;
                for (int64_t k = 0; k < K; k++) ss += (double)x[k] * (double)x[k];
                const double c = 1.0 / sqrt(ss / (double)K + (double)norm_eps);
                for (int64_t k = 0; k < K; k++) t += (gain ? (double)gain[k] : 1.0) * dr[k] * (double)x[k];
                for (int64_t k = 0; k < K; k++)
                    out[k] = c * (gain ? (double)gain[k] : 1.0) * dr[k] - c * c * c / (double)K * (double)x[k] * t;
            } else {
                double mu = 0.0, var = 0.0, ma = 0.0, max_ = 0.0;
                for (int64_t k = 0; k < K; k++) mu += (double)x[k];
                mu = mu / (double)K;
                for (int64_t k = 0; k < K; k++) var += ((double)x[k] - mu) * ((double)x[k] - mu);
                const double c = 1.0 / sqrt(var / (double)K + (double)norm_eps);
                for (int64_t k = 0; k < K; k++) {
                    const double a = (gain ? (double)gain[k] : 1.0) * dr[k];
                    ma += a;
                    max_ += a * ((double)x[k] - mu) * c;
                }
                ma /= (double)K;
                max_ /= (double)K;
                for (int64_t k = 0; k < K; k++) {
                    const double a = (gain ? (double)gain[k] : 1.0) * dr[k];
                    out[k] = c * (a - ma - ((double)x[k] - mu) * c * max_);
                }
            }
        }
        if (dW) {
            rc = hbo_quantize_activations(X, M, K, gain, norm, norm_eps, hadamard, bits, a4_mode, quant_eps, NULL, q,
                                          s, d);
            if (rc == HBO_OK) hbo_weight_grad(dY, q, d, M, N, K, dW);
        }
    }
    free(dz); free(dr); free(q); free(s); free(d);
    return rc;
}

/* --------------------------------------------------------------- O13 ---- */
/* Base-3 weight storage.  [CSDN] "掩码存储" lists two ways of storing ternary
 * weights; the first packs several weights into one integer, five per 8-bit
 * byte (3^5 = 243 <= 256, 1.6 bits per weight).  The digit order and the row
 * layout are not given; the reading taken: byte j of row n holds the weights
 * k = 5j .. 5j+4 as base-3 digits t + 1 (t in {-1, 0, +1}), the first weight
 * least significant,
 *   byte = sum_{i=0..4} (W_q[n][5j+i] + 1) * 3^i,
 * weights past K count as 0 (digit 1), and every row is padded to a whole
 * number of 16-byte vectors: 16 * ceil(K / 80) bytes.  Bytes 243..255 never
 * occur. */
int64_t hbo_base3_row_bytes(int64_t K) { return 16 * ((K + 79) / 80); }

int hbo_pack_base3(const int8_t* Wq, int64_t N, int64_t K, uint8_t* out) {
    if (N < 0 || K < 1) return HBO_ERR;
    const int64_t RB = hbo_base3_row_bytes(K);
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < RB; j++) {
            int v = 0, place = 1;
            for (int i = 0; i < 5; i++) {
                const int64_t k = 5 * j + i;
                const int t = k < K ? Wq[n * K + k] : 0;
                if (t < -1 || t > 1) return HBO_ERR;
                v += (t + 1) * place;
                place *= 3;
            }
            out[n * RB + j] = (uint8_t)v;
        }
    return HBO_OK;
}

/* The inverse: base-3 digits of each byte, least significant first, minus 1.
 * A byte above 242, or a padding weight that is not 0, is an error. */
int hbo_unpack_base3(const uint8_t* in, int64_t N, int64_t K, int8_t* Wq) {
    if (N < 0 || K < 1) return HBO_ERR;
    const int64_t RB = hbo_base3_row_bytes(K);
    for (int64_t n = 0; n < N; n++)
        for (int64_t j = 0; j < RB; j++) {
            int v = in[n * RB + j];
            if (v > 242) return HBO_ERR;
            for (int i = 0; i < 5; i++) {
                const int t = v % 3 - 1;
                v /= 3;
                const int64_t k = 5 * j + i;
                if (k < K) Wq[n * K + k] = (int8_t)t;
                else if (t != 0) return HBO_ERR;
            }
        }
    return HBO_OK;
}

/* --------------------------------------------------------------- O14 ---- */
/* FP4 weight storage for the INT4 prefill path on FP6 x FP4 matrix hardware
 * ([XZY] "原生4比特盘算": 4-bit activations suit native low-bit compute; the
 * format is the library's own).  W4 [N][K/2]: weight k of row n in byte k/2,
 * the low nibble for even k.  The nibble is the E2M1 encoding of the ternary
 * value: sign in bit 3, a 2-bit exponent with bias 1 in bits 2..1, one
 * mantissa bit in bit 0; so 0 -> 0000, +1.0 -> 0010 (exponent 1, mantissa
 * 0), -1.0 -> 1010.  Requires K even. */
int hbo_pack_fp4(const int8_t* Wq, int64_t N, int64_t K, uint8_t* W4) {
    if (N < 0 || K < 2 || K % 2) return HBO_ERR;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k += 2) {
            uint8_t b = 0;
            for (int h = 0; h < 2; h++) {
                const int t = Wq[n * K + k + h];
                uint8_t code;
                if (t == 0) code = 0x0;
                else if (t == 1) code = 0x2;
                else if (t == -1) code = 0xA;
                else return HBO_ERR;
                b |= (uint8_t)(code << (4 * h));
            }
            W4[n * (K / 2) + k / 2] = b;
        }
    return HBO_OK;
}
