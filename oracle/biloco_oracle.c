/*
 * biloco_oracle.c -- plain, slow, fp64 CPU oracle for the BiLoCo fused product
 *
 *     y = Q4(x) . deq(R)^T  +  sum_i alpha_i (x . v_i) u_i
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant generator with the HIP library; every routine below is written
 * from the format definitions and from the method's statement on the pages.
 *
 * Sources (the pages the method is described on):
 *   [BiLoCo]  "BiLoCo: Binary Low-Rank Corrections for Post-Training
 *             Quantization" (project README).  Intro: W ~ U diag(alpha) V^T + R,
 *             U, V sign matrices, R in NVFP4.  Section "Kernel": the fused
 *             product y = FP4(x) FP4(R)^T + sum_i alpha_i (x.v_i) u_i, decode
 *             batches up to 32, z = alpha (.) (V x) from packed V signs,
 *             expansion of z through packed U signs before the BF16 store, and
 *             the operand list of the launcher (codes, block scales, global
 *             scale, pack_signs(V.T), pack_signs(U.T), alpha.bfloat16(), x).
 *   NVFP4 as used here: E2M1 element codes, one E4M3 scale per 16 elements
 *   along K, an fp32 global scale on the residual R; activation scale is
 *   E4M3(amax/6) with codes rounded to nearest-even.
 *
 * Every function is the plain definition: nearest-value searches for the
 * two roundings, straight triple loops in double for the products.  Where
 * the pages leave a step open the reading taken is stated at the function.
 *
 * Parity pins: every function here is pinned by the CPU test-suite against
 * an independent route (library casts, numpy matmul, dense reconstruction,
 * closed forms, exhaustive brute force).  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Element formats                                                     */
/* ------------------------------------------------------------------ */

/* E2M1 (FP4) value of a 4-bit code: bit 3 sign, bits 2..1 exponent (bias 1),
 * bit 0 mantissa; exponent field 0 is subnormal with value 0.5*m. */
double oracle_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E4M3 (OCP "FN" variant) value of a byte: bit 7 sign, bits 6..3 exponent
 * (bias 7), bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); the
 * single pattern S.1111.111 is NaN; there is no infinity; max is 448. */
double oracle_e4m3_value(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Round a non-negative finite value to E4M3: the nearest finite E4M3 value,
 * ties to the code with an even mantissa (low bit 0).  Values beyond the
 * largest finite value 448 saturate to it (0x7E): the pages do not say what
 * overflow does and this path never reaches it.  Returns the byte. */
unsigned oracle_e4m3_encode(double v)
{
    unsigned best = 0, b;
    double bestd = INFINITY;
    if (!(v >= 0.0)) v = 0.0;          /* negative / NaN never asked for */
    if (v >= 448.0) return 0x7Eu;
    for (b = 0; b < 0x7Fu; ++b) {      /* all finite non-negative codes */
        double d = fabs(oracle_e4m3_value(b) - v);
        if (d < bestd || (d == bestd && (b & 1u) == 0u)) { bestd = d; best = b; }
    }
    return best;
}

/* Round x/s to E2M1 for a block scale s > 0: the nearest of the eight
 * magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} to |x|/s, ties to the even code,
 * saturating at 6; the sign bit is the sign of x (so a negative value that
 * rounds to zero gives code 8).  With s == 0 the magnitude is 0. */
unsigned oracle_e2m1_encode(double x, double s)
{
    unsigned sign = signbit(x) ? 8u : 0u, c, best = 0;
    double t, bestd = INFINITY;
    if (s == 0.0) return sign;
    t = fabs(x) / s;
    if (t > 6.0) t = 6.0;              /* saturate before measuring distances */
    for (c = 0; c < 8; ++c) {
        double d = fabs(oracle_e2m1_value(c) - t);
        if (d < bestd || (d == bestd && (c & 1u) == 0u)) { bestd = d; best = c; }
    }
    return sign | best;
}

/* Element-wise E2M1 rounding of n (x, s) pairs (the function above in a loop;
 * lets the tests sweep millions of pairs without a call per pair). */
void oracle_e2m1_encode_n(const double *x, const double *s, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e2m1_encode(x[i], s[i]);
}

/* Element-wise E4M3 rounding of n non-negative values. */
void oracle_e4m3_encode_n(const double *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_encode(v[i]);
}

/* bfloat16 bits -> value (exact). */
double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------ */
/* Activation FP4 quantisation                                          */
/* ------------------------------------------------------------------ */

/* x: bf16 [M][K] row-major, K a multiple of 16.
 * Per row m and block b of 16 consecutive k:
 *   amax = max |x|;  s = E4M3(amax / 6);  code_k = E2M1(x_k / value(s)).
 * Outputs: codes [M][K/2], element k in the low nibble of byte k/2 when k is
 * even and in the high nibble when k is odd; scales [M][K/16], one E4M3 byte
 * per block.  [BiLoCo, "Kernel": the activation operand is NVFP4 codes plus
 * block scales; the amax/6 rule and nearest-even codes are the workload's.] */
void oracle_quant_act_fp4(const uint16_t *x, int64_t M, int64_t K,
                          uint8_t *codes, uint8_t *scales)
{
    int64_t m, b, j;
    for (m = 0; m < M; ++m) {
        for (b = 0; b < K / 16; ++b) {
            double amax = 0.0, s;
            unsigned sbyte;
            for (j = 0; j < 16; ++j) {
                double v = fabs(oracle_bf16_value(x[m * K + b * 16 + j]));
                if (v > amax) amax = v;
            }
            sbyte = oracle_e4m3_encode(amax / 6.0);
            scales[m * (K / 16) + b] = (uint8_t)sbyte;
            s = oracle_e4m3_value(sbyte);
            for (j = 0; j < 16; j += 2) {
                int64_t k = b * 16 + j;
                unsigned lo = oracle_e2m1_encode(oracle_bf16_value(x[m * K + k]), s);
                unsigned hi = oracle_e2m1_encode(oracle_bf16_value(x[m * K + k + 1]), s);
                codes[(m * K + k) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* NVFP4 weight quantisation of the residual R                          */
/* ------------------------------------------------------------------ */

/* w: fp32 [N][K] row-major, K a multiple of 16, finite values.
 * [BiLoCo, intro and "Decomposition": R is stored in NVFP4; "Kernel": the
 * launcher takes its codes, its block scales and an fp32 global scale.  The
 * pages give no recipe; the reading taken here is the plain one in which the
 * largest block scale lands on the largest E4M3 value:]
 *   amax = max |w|;  g = fp32(amax / (6 * 448))  (g = 1 when amax == 0)
 *   per row n, block b of 16 consecutive k:
 *     a = max |w| over the block;  t = fp32(a / 6);  q = fp32(t / g)
 *     scale byte s = E4M3(q), nearest, ties to even, saturating at 448
 *     d = fp32(value(s) * g)
 *     code_k = E2M1 nearest to fp32(|w_k| / d), ties to the even code,
 *              saturating at 6, sign of w_k kept; d == 0 gives signed zero
 * so that w_k ~ g * value(s) * e2m1(code_k).  Every fp32(...) above is one
 * correctly rounded single-precision operation (C float arithmetic).
 * Outputs: codes [N][K/2] (even k in the low nibble), scales [N][K/16], *g. */
void oracle_quant_weight_nvfp4(const float *w, int64_t N, int64_t K,
                               uint8_t *codes, uint8_t *scales, float *g_out)
{
    int64_t n, b, j, total = N * K;
    float amax = 0.0f, g;
    for (j = 0; j < total; ++j) {
        float a = fabsf(w[j]);
        if (a > amax) amax = a;
    }
    g = amax > 0.0f ? amax / 2688.0f : 1.0f;
    *g_out = g;
    for (n = 0; n < N; ++n) {
        for (b = 0; b < K / 16; ++b) {
            const float *blk = w + n * K + b * 16;
            float a = 0.0f, t, q, d;
            unsigned sbyte;
            for (j = 0; j < 16; ++j)
                if (fabsf(blk[j]) > a) a = fabsf(blk[j]);
            t = a / 6.0f;
            q = t / g;
            sbyte = oracle_e4m3_encode((double)q);
            scales[n * (K / 16) + b] = (uint8_t)sbyte;
            d = (float)oracle_e4m3_value(sbyte) * g;
            for (j = 0; j < 16; j += 2) {
                unsigned c[2], h;
                for (h = 0; h < 2; ++h) {
                    float x = blk[j + h];
                    unsigned sign = signbit(x) ? 8u : 0u;
                    if (d == 0.0f) { c[h] = sign; continue; }
                    {
                        float tq = fabsf(x) / d;
                        c[h] = sign | oracle_e2m1_encode((double)tq, 1.0);
                    }
                }
                codes[(n * K + b * 16 + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Sign packing                                                         */
/* ------------------------------------------------------------------ */

/* signs: int8 [rows][cols] row-major (the caller passes V^T or U^T, so rows
 * is the rank axis).  Output words [ceil(rows/32)][cols]: bit b of word
 * (w, c) is 1 when signs[32w+b][c] < 0; bits for 32w+b >= rows are 0.
 * [BiLoCo, "Kernel": the launcher takes pack_signs(V.T), pack_signs(U.T);
 * the workload packs 32 signs per uint32 along r.] */
void oracle_pack_signs(const int8_t *signs, int64_t rows, int64_t cols, uint32_t *packed)
{
    int64_t W = (rows + 31) / 32, w, c, b;
    for (w = 0; w < W; ++w)
        for (c = 0; c < cols; ++c) {
            uint32_t word = 0;
            for (b = 0; b < 32; ++b) {
                int64_t row = w * 32 + b;
                if (row < rows && signs[row * cols + c] < 0) word |= (uint32_t)1u << b;
            }
            packed[w * cols + c] = word;
        }
}

/* ------------------------------------------------------------------ */
/* The fused product, in double                                         */
/* ------------------------------------------------------------------ */

/* Inputs (method-level operands, not the kernel's packed forms):
 *   x      bf16 [M][K]            activation
 *   wcode  uint8 [N][K]           one E2M1 code (0..15) per element of R
 *   wscale uint8 [N][K/16]        E4M3 block scales of R
 *   g      float                  global scale of R
 *   V      int8 [K][r]  (+1/-1)   right sign factor
 *   U      int8 [N][r]  (+1/-1)   left sign factor
 *   alpha  bf16 [r]               coefficients (the launcher takes bf16)
 * Outputs (any may be NULL):
 *   y      double [M][N]   G + C
 *   gpart  double [M][N]   G = g * Q4(x) deq(R)^T
 *   cpart  double [M][N]   C = sum_i z[m][i] U[n][i]
 *   z      double [M][r]   z[m][i] = alpha_i * sum_k x[m][k] V[k][i]
 * Readings: the correction uses the unquantised bf16 x (the launcher passes
 * x next to the FP4 activation and the formula applies FP4 only to the
 * first term); z = alpha (.) (x V) with V stored [K][r]; g scales R only.
 * Q4(x) is this file's own quantiser above. */
void oracle_gemm_lowrank(const uint16_t *x, const uint8_t *wcode, const uint8_t *wscale,
                         float g, const int8_t *V, const int8_t *U, const uint16_t *alpha,
                         int64_t M, int64_t N, int64_t K, int64_t r,
                         double *y, double *gpart, double *cpart, double *z)
{
    int64_t KB = K / 16;
    uint8_t *acode = (uint8_t *)malloc((size_t)(M * K / 2 > 0 ? M * K / 2 : 1));
    uint8_t *ascale = (uint8_t *)malloc((size_t)(M * KB > 0 ? M * KB : 1));
    double *A = (double *)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double *zz = (double *)malloc(sizeof(double) * (size_t)(M * r > 0 ? M * r : 1));
    int64_t m, k;
    oracle_quant_act_fp4(x, M, K, acode, ascale);

    /* A = Q4(x) dequantised: code value times its block's scale value */
    for (m = 0; m < M; ++m)
        for (k = 0; k < K; ++k) {
            unsigned byte = acode[(m * K + k) / 2];
            unsigned c = (k & 1) ? (byte >> 4) : (byte & 15u);
            A[m * K + k] = oracle_e2m1_value(c) * oracle_e4m3_value(ascale[m * KB + k / 16]);
        }

    /* z[m][i] = alpha_i * sum_k x[m][k] * V[k][i] */
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t mi = 0; mi < M * r; ++mi) {
        int64_t mm = mi / r, ii = mi % r, kk;
        double acc = 0.0;
        for (kk = 0; kk < K; ++kk) acc += oracle_bf16_value(x[mm * K + kk]) * (double)V[kk * r + ii];
        zz[mm * r + ii] = oracle_bf16_value(alpha[ii]) * acc;
    }

    /* per output column n: G from the dequantised R row n, C from z and U's
     * row n.  The row of deq(R) is decoded once into a scratch row and then
     * used for every m (the same products, only not decoded M times). */
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        double *B = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t n = 0; n < N; ++n) {
            int64_t mm, kk, ii;
            for (kk = 0; kk < K; ++kk)
                B[kk] = oracle_e2m1_value(wcode[n * K + kk]) * oracle_e4m3_value(wscale[n * KB + kk / 16]);
            for (mm = 0; mm < M; ++mm) {
                double gacc = 0.0, cacc = 0.0, gv;
                for (kk = 0; kk < K; ++kk) gacc += A[mm * K + kk] * B[kk];
                gv = (double)g * gacc;
                for (ii = 0; ii < r; ++ii) cacc += zz[mm * r + ii] * (double)U[n * r + ii];
                if (gpart) gpart[mm * N + n] = gv;
                if (cpart) cpart[mm * N + n] = cacc;
                if (y) y[mm * N + n] = gv + cacc;
            }
        }
        free(B);
    }
    if (z) memcpy(z, zz, sizeof(double) * (size_t)(M * r));
    free(acode); free(ascale); free(A); free(zz);
}

/* Number of threads the parallel loop above uses (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops from now on (timing runs: all host cores,
 * then one).  No effect on any result: every output is computed by one
 * thread in a fixed order. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
