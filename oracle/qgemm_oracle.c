/*
 * qgemm_oracle.c -- plain CPU oracle for the scaled low-precision GEMM
 *
 *     C = bf16( scale_A (.) scale_B (.) (A . B^T) + bias )
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no header, table or helper with the HIP path.
 *
 * Sources, by page title and section:
 *  - "Optimize HIP WMMA INT8 GEMM staging, epilogue, and deep-K tiling"
 *    (comfy-kitchen PR #174): Summary (rowwise scales and bias; signed zero
 *    kept without bias), Validation (int8 results exact), Update "rebased
 *    onto v0.2.40" (association pinned to (acc*sa)*sb).
 *  - "perf(gemm-ar): mxfp8 with row-major scales staged through LDS"
 *    (ROCm/mori PR #806): What (32-wide ue8m0 scales; A scales [M,K/32], B
 *    scales [N/32,K/32] uint8 row-major), Measured (per-token/per-channel
 *    "ptpc" FP8).
 *  - "[fp4_gemm_4wave] MXFP4 GEMM perf optimize" (ROCm/FlyDSL PR #990):
 *    MXFP4 = e2m1 elements with one ue8m0 scale per 1x32 K block.
 * The pages name e4m3 / e2m1 / ue8m0 without giving their bits; the reading
 * taken is the OCP 8-bit floating point (E4M3FN) and OCP Microscaling v1.0
 * definitions of those names.
 *
 * Arithmetic: integers accumulate exactly (int64, checked to fit int32, the
 * accumulator the INT8 page specifies); e4m3 / e2m1 / ue8m0 are decoded
 * exactly to double and accumulated in double (every sum here is exact for
 * these formats up to the bounds stated per function); the epilogue is a
 * fixed sequence of IEEE binary32 operations, each rounded to nearest even,
 * subnormals kept, no fused multiply-add (built with -ffp-contract=off), and
 * a final round-to-nearest-even to bfloat16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* E4M3FN: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent field 0
 * is subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity, and the
 * largest finite magnitude is 1.75 * 2^8 = 448. */
double orc_dec_e4m3(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent field 0 is
 * subnormal (m * 0.5); every code is finite, largest magnitude 6. */
double orc_dec_e2m1(uint8_t nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double v = (e == 0) ? 0.5 * m : ldexp((double)(2 + m), e - 2);
    return s ? -v : v;
}

/* FP6 E2M3 (OCP Microscaling v1.0): sign (bit 5), 2-bit exponent (bias 1),
 * 3-bit mantissa; exponent field 0 is subnormal (m * 2^-3); every code is
 * finite; the largest magnitude is 1.875 * 2^2 = 7.5. */
double orc_dec_e2m3(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -3) : ldexp((double)(8 + m), e - 4);
    return s ? -v : v;
}

/* FP6 E3M2 (OCP Microscaling v1.0): sign (bit 5), 3-bit exponent (bias 3),
 * 2-bit mantissa; exponent field 0 is subnormal (m * 2^-4); every code is
 * finite; the largest magnitude is 1.75 * 2^4 = 28. */
double orc_dec_e3m2(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 2) & 7, m = code & 3;
    double v = (e == 0) ? ldexp((double)m, -4) : ldexp((double)(4 + m), e - 5);
    return s ? -v : v;
}

/* E8M0 (unsigned, exponent only, bias 127): code c is 2^(c-127), 255 is NaN. */
double orc_dec_ue8m0(uint8_t code)
{
    if (code == 255)
        return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* bfloat16 bits -> binary32 (exact: bf16 is the upper half of binary32). */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays NaN (quiet,
 * sign kept); overflow rounds to infinity as IEEE rounding does. */
uint16_t orc_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ INT8 */

/* INT8 rowwise GEMM.  A [M,K] int8 (row stride lda), B [N,K] int8 (row
 * stride ldb), scale_a [M] and scale_b [N] binary32, bias [N] bf16 bits or
 * NULL, C [M,ldc] bf16 bits.  acc (optional, [M,N] dense) receives the int32
 * accumulator.  Returns 0, or -1 if an accumulator leaves the int32 range
 * (impossible for K <= 131071).
 *
 * Per output: acc = sum_k A[m,k]*B[n,k] exactly; f = (float)acc;
 * f = f*sa[m]; f = f*sb[n]; if bias: f = f + bias[n]; C = bf16_rne(f).
 * Without bias nothing is added, so a -0 product stays -0. */
int orc_i8_rowwise(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                   const float *scale_a, const float *scale_b, const uint16_t *bias,
                   uint16_t *C, int64_t ldc, int32_t *acc,
                   int64_t M, int64_t N, int64_t K)
{
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *a = A + m * lda;
            const int8_t *b = B + n * ldb;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int32_t)a[k] * (int32_t)b[k];
            if (s > INT32_MAX || s < INT32_MIN)
                bad = 1;
            int32_t s32 = (int32_t)s;
            if (acc)
                acc[m * N + n] = s32;
            float f = (float)s32;
            f = f * scale_a[m];
            f = f * scale_b[n];
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ FP8 */

/* FP8 e4m3 per-token (row of A) / per-channel (row of B) GEMM.  A [M,K] and
 * B [N,K] e4m3 codes, scale_a [M] / scale_b [N] binary32, bias as above.
 * acc (optional [M,N]) receives the double accumulator; absdot (optional
 * [M,N]) receives |sa[m]*sb[n]| * sum_k |a_k*b_k|, the scale of the error
 * bound.
 *
 * Every e4m3 value is an integer multiple of 2^-9 of magnitude at most
 * 448 = 229376 * 2^-9, so each product is a multiple of 2^-18 below 2^35.7
 * and a sum of K <= 131072 such products stays below 2^53 * 2^-18: the
 * double sum is exact, whatever its order.
 *
 * Per output: f = (float)acc; f = f*sa[m]; f = f*sb[n]; [f = f + bias[n]];
 * C = bf16_rne(f). */
void orc_f8_pertoken(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                     const float *scale_a, const float *scale_b, const uint16_t *bias,
                     uint16_t *C, int64_t ldc, double *acc, double *absdot,
                     int64_t M, int64_t N, int64_t K)
{
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = orc_dec_e4m3((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *a = A + m * lda;
            const uint8_t *b = B + n * ldb;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = lut[a[k]] * lut[b[k]];
                s += p;
                t += fabs(p);
            }
            if (acc)
                acc[m * N + n] = s;
            if (absdot)
                absdot[m * N + n] = fabs((double)scale_a[m] * (double)scale_b[n]) * t;
            float f = (float)s;
            f = f * scale_a[m];
            f = f * scale_b[n];
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
}

/* ------------------------------------------------------------------- MX */

/* MX GEMM: fmt 0 = e4m3 elements (one byte each), fmt 1 = e2m1 elements (two
 * per byte, element k in the low nibble of byte k/2 when k is even, in the
 * high nibble when k is odd).  lda / ldb are row strides in BYTES.
 * scale_a: ue8m0 codes [M, K/32] row-major (row stride K/32).
 * scale_b: ue8m0 codes, b_rows_per_scale = 1 -> [N, K/32] (one scale per row
 * of B and K block), = 32 -> [ceil(N/32), K/32] (one scale per 32 rows of B
 * and K block).  bias / C as above; acc / absdot as for FP8, here over the
 * scaled values (absdot = sum_k |A~[m,k] * B~[n,k]|).
 *
 * A~[m,k] = dec(A[m,k]) * 2^(SA[m,k/32]-127) and likewise B~; each is exact in
 * double (a power-of-two multiple of a short integer).  acc = sum_k A~ B~ in
 * double; with the power-of-two scales the terms of one row pair differ only
 * by the spread of their scale exponents, and for spreads within the bound
 * the tests check (an exact integer recomputation) the sum is exact.
 *
 * Per output: f = (float)acc; [f = f + bias[n]]; C = bf16_rne(f).
 * Returns 0, or -1 for an unknown fmt / b_rows_per_scale. */
int orc_mx(int fmt, const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
           const uint8_t *scale_a, const uint8_t *scale_b, int b_rows_per_scale,
           const uint16_t *bias, uint16_t *C, int64_t ldc, double *acc, double *absdot,
           int64_t M, int64_t N, int64_t K)
{
    if ((fmt != 0 && fmt != 1) || (b_rows_per_scale != 1 && b_rows_per_scale != 32))
        return -1;
    const int64_t KB = K / 32;
    double lut8[256], lut4[16], lut_s[256];
    for (int c = 0; c < 256; ++c) {
        lut8[c] = orc_dec_e4m3((uint8_t)c);
        lut_s[c] = orc_dec_ue8m0((uint8_t)c);
    }
    for (int c = 0; c < 16; ++c)
        lut4[c] = orc_dec_e2m1((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *sarow = scale_a + m * KB;
            const uint8_t *sbrow = scale_b + (n / b_rows_per_scale) * KB;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a, b;
                if (fmt == 0) {
                    a = lut8[A[m * lda + k]];
                    b = lut8[B[n * ldb + k]];
                } else {
                    uint8_t ab = A[m * lda + k / 2], bb = B[n * ldb + k / 2];
                    a = lut4[(k & 1) ? (ab >> 4) : (ab & 15)];
                    b = lut4[(k & 1) ? (bb >> 4) : (bb & 15)];
                }
                a *= lut_s[sarow[k / 32]];
                b *= lut_s[sbrow[k / 32]];
                double p = a * b;
                s += p;
                t += fabs(p);
            }
            if (acc)
                acc[m * N + n] = s;
            if (absdot)
                absdot[m * N + n] = t;
            float f = (float)s;
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
    return 0;
}

/* MX GEMM with its own element format per operand: fmt_a for A, fmt_b for B
 * (0 = e4m3, one byte per element; 1 = e2m1, two per byte as in orc_mx).  The
 * MX scale rule of "perf(gemm-ar): mxfp8 with row-major scales staged through
 * LDS" (ROCm/mori PR #806, What) and "[fp4_gemm_4wave] MXFP4 GEMM perf
 * optimize" (ROCm/FlyDSL PR #990) applies to each operand unchanged: one ue8m0
 * scale per 32 elements along K, A scales [M, K/32], B scales [N, K/32] or
 * [ceil(N/32), K/32].  With fmt_a == fmt_b this is orc_mx.  Each product
 * A~ B~ is exact in double; the sum is exact under the same bound as orc_mx
 * (an e4m3 x e2m1 product is a multiple of 2^-10 below 2^11.4).
 * Returns 0, or -1 for an unknown format / b_rows_per_scale. */
int orc_mx2(int fmt_a, int fmt_b, const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
            const uint8_t *scale_a, const uint8_t *scale_b, int b_rows_per_scale,
            const uint16_t *bias, uint16_t *C, int64_t ldc, double *acc, double *absdot,
            int64_t M, int64_t N, int64_t K)
{
    if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1) ||
        (b_rows_per_scale != 1 && b_rows_per_scale != 32))
        return -1;
    const int64_t KB = K / 32;
    double lut8[256], lut4[16], lut_s[256];
    for (int c = 0; c < 256; ++c) {
        lut8[c] = orc_dec_e4m3((uint8_t)c);
        lut_s[c] = orc_dec_ue8m0((uint8_t)c);
    }
    for (int c = 0; c < 16; ++c)
        lut4[c] = orc_dec_e2m1((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *sarow = scale_a + m * KB;
            const uint8_t *sbrow = scale_b + (n / b_rows_per_scale) * KB;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a, b;
                if (fmt_a == 0) {
                    a = lut8[A[m * lda + k]];
                } else {
                    const uint8_t ab = A[m * lda + k / 2];
                    a = lut4[(k & 1) ? (ab >> 4) : (ab & 15)];
                }
                if (fmt_b == 0) {
                    b = lut8[B[n * ldb + k]];
                } else {
                    const uint8_t bb = B[n * ldb + k / 2];
                    b = lut4[(k & 1) ? (bb >> 4) : (bb & 15)];
                }
                a *= lut_s[sarow[k / 32]];
                b *= lut_s[sbrow[k / 32]];
                const double p = a * b;
                s += p;
                t += fabs(p);
            }
            if (acc)
                acc[m * N + n] = s;
            if (absdot)
                absdot[m * N + n] = t;
            float f = (float)s;
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
    return 0;
}

/* ------------------------------------------ MX, any element format */

/* Element k of an MX operand row in format fmt, as its code:
 *   0 e4m3: byte k;
 *   1 e2m1: the low nibble of byte k/2 when k is even, the high one when odd;
 *   2 e2m3, 3 e3m2 (6-bit): bits 6k .. 6k+5 of the row read as one bit string
 *     whose bit b is bit (b mod 8) of byte b/8 -- four elements in three
 *     bytes, the lowest bits first, as e2m1 keeps its even element in the
 *     low nibble. */
static unsigned mx_code(const uint8_t *row, int64_t k, int fmt)
{
    if (fmt == 0)
        return row[k];
    if (fmt == 1)
        return (k & 1) ? (row[k / 2] >> 4) : (row[k / 2] & 15);
    const int64_t bit = 6 * k;
    const int sh = (int)(bit & 7);
    unsigned v = (unsigned)row[bit >> 3] >> sh;
    if (sh > 2)
        v |= (unsigned)row[(bit >> 3) + 1] << (8 - sh);
    return v & 63;
}

/* Bytes of an MX operand row of K elements in format fmt. */
int64_t orc_mx_row_bytes(int fmt, int64_t K)
{
    return fmt == 0 ? K : fmt == 1 ? K / 2 : 3 * K / 4;
}

/* MX GEMM with an element format per operand, any of e4m3 (0), e2m1 (1) and
 * the two 6-bit formats e2m3 (2) and e3m2 (3) that OCP Microscaling v1.0
 * defines next to them (the pages name MX e4m3 and e2m1; MXFP6 is the same
 * block rule with 6-bit elements).  Element layout as mx_code; lda / ldb are
 * row strides in bytes; scales, bias, acc, absdot and the epilogue as orc_mx:
 *
 *   A~[m,k] = dec(A[m,k]) * 2^(SA[m,k/32]-127), B~ likewise,
 *   acc = sum_k A~ B~ (double), f = (float)acc; [f = f + bias[n]];
 *   C = bf16_rne(f).
 *
 * Every 6-bit value is a multiple of 2^-3 (e2m3) or 2^-4 (e3m2) of magnitude
 * at most 7.5 or 28, so each product is exact in double and the sum is exact
 * under the scale-spread bound of orc_mx.  K must be a multiple of 32 (of 4
 * for whole bytes of 6-bit rows, which 32 implies).
 * Returns 0, or -1 for an unknown format / b_rows_per_scale. */
int orc_mxf(int fmt_a, int fmt_b, const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
            const uint8_t *scale_a, const uint8_t *scale_b, int b_rows_per_scale,
            const uint16_t *bias, uint16_t *C, int64_t ldc, double *acc, double *absdot,
            int64_t M, int64_t N, int64_t K)
{
    if (fmt_a < 0 || fmt_a > 3 || fmt_b < 0 || fmt_b > 3 || (b_rows_per_scale != 1 && b_rows_per_scale != 32) ||
        K % 32 != 0)
        return -1;
    const int64_t KB = K / 32;
    double lut[4][256], lut_s[256];
    for (int c = 0; c < 256; ++c) {
        lut[0][c] = orc_dec_e4m3((uint8_t)c);
        lut[1][c] = c < 16 ? orc_dec_e2m1((uint8_t)c) : 0.0;
        lut[2][c] = c < 64 ? orc_dec_e2m3((uint8_t)c) : 0.0;
        lut[3][c] = c < 64 ? orc_dec_e3m2((uint8_t)c) : 0.0;
        lut_s[c] = orc_dec_ue8m0((uint8_t)c);
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *arow = A + m * lda, *brow = B + n * ldb;
            const uint8_t *sarow = scale_a + m * KB;
            const uint8_t *sbrow = scale_b + (n / b_rows_per_scale) * KB;
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = lut[fmt_a][mx_code(arow, k, fmt_a)] * lut_s[sarow[k / 32]];
                const double b = lut[fmt_b][mx_code(brow, k, fmt_b)] * lut_s[sbrow[k / 32]];
                const double p = a * b;
                s += p;
                t += fabs(p);
            }
            if (acc)
                acc[m * N + n] = s;
            if (absdot)
                absdot[m * N + n] = t;
            float f = (float)s;
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
    return 0;
}

/* ------------------------------------------------------- FP8 blockscale */

/* FP8 e4m3 GEMM with block-wise fp32 scales: the "blockscale" variant that
 * "perf(gemm-ar): mxfp8 with row-major scales staged through LDS" (ROCm/mori
 * PR #806) measures next to per-token FP8 and MXFP8 (commit message table,
 * M=16384 N=7168 K=2048).  The page names the variant but not its blocks;
 * the reading taken: K is cut into blocks of 128 elements, A has one scale
 * per row and K block (scale_a [M, K/128], row stride K/128) and B one per
 * 128 rows and K block (scale_b [ceil(N/128), K/128]), both binary32 and
 * row-major, so that
 *
 *     C[m,n] = bf16( sum_kb sa[m,kb] * sb[n/128,kb] * P[m,n,kb] (+ bias[n]) ),
 *     P[m,n,kb] = sum over the block's k of dec(A[m,k]) * dec(B[n,k]).
 *
 * P is exact in double (at most 128 products, each a multiple of 2^-18 below
 * 2^35.7); sa*sb is exact in double (two 24-bit significands); each term
 * sa*sb*P and the sum over blocks round once in double, so acc lies within
 * (K/128 + 1) * 2^-53 * absdot of the exact sum, far inside the GEMM's
 * tolerance.  acc / absdot as for FP8 (absdot = sum_k |sa sb a_k b_k|).
 * K must be a multiple of 128.
 *
 * Per output: f = (float)acc; [f = f + bias[n]]; C = bf16_rne(f).
 * Returns 0, or -1 if K is not a multiple of 128. */
int orc_f8_blockscale(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                      const float *scale_a, const float *scale_b, const uint16_t *bias,
                      uint16_t *C, int64_t ldc, double *acc, double *absdot,
                      int64_t M, int64_t N, int64_t K)
{
    if (K % 128 != 0)
        return -1;
    const int64_t KB = K / 128;
    double lut[256];
    for (int c = 0; c < 256; ++c)
        lut[c] = orc_dec_e4m3((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *a = A + m * lda;
            const uint8_t *b = B + n * ldb;
            const float *sarow = scale_a + m * KB;
            const float *sbrow = scale_b + (n / 128) * KB;
            double s = 0.0, t = 0.0;
            for (int64_t kb = 0; kb < KB; ++kb) {
                double p = 0.0, q = 0.0;
                for (int64_t k = 128 * kb; k < 128 * kb + 128; ++k) {
                    double x = lut[a[k]] * lut[b[k]];
                    p += x;
                    q += fabs(x);
                }
                double w = (double)sarow[kb] * (double)sbrow[kb];
                s += w * p;
                t += fabs(w) * q;
            }
            if (acc)
                acc[m * N + n] = s;
            if (absdot)
                absdot[m * N + n] = t;
            float f = (float)s;
            if (bias)
                f = f + orc_bf16_to_f32(bias[n]);
            C[m * ldc + n] = orc_bf16_rne(f);
        }
    }
    return 0;
}

/* ----------------------------------------------------------- quantisers */

/* The quantisers that produce the GEMM's operands from bf16 activations.
 * "perf(gemm-ar): mxfp8 with row-major scales staged through LDS" (ROCm/mori
 * PR #806), What: the quantiser hands the GEMM its A scales as [M, K/32]
 * uint8 ue8m0 codes, row-major; Measured: per-token ("ptpc") e4m3 scales.
 * The pages give no formula for either scale.  The readings taken:
 *  - per-token e4m3: scale[m] = fp32(amax_m / 448), 448 being the largest
 *    finite e4m3 magnitude, and code = enc(fp32(x / scale[m])); an all-zero
 *    row gets scale 0 and keeps each zero's sign;
 *  - MX: the OCP Microscaling v1.0 scale rule, shared exponent
 *    X = floor(log2(amax)) - emax (emax 8 for e4m3, 2 for e2m1), stored as
 *    the ue8m0 code X + 127 clamped to [0, 254] (0 for an all-zero block),
 *    and code = enc(x * 2^-(code - 127));
 *  - enc: the nearest representable magnitude, ties to the even code,
 *    magnitudes beyond the largest finite one saturating to it; the sign bit
 *    is x's sign bit (so a negative value that rounds to zero is -0).
 * Inputs are finite; for NaN or infinite inputs the result is unspecified. */

/* Nearest of the first ncodes magnitudes dec(0) < dec(1) < ... to a >= 0:
 * a plain walk up the decoded grid. */
static int enc_nearest(double a, double (*dec)(uint8_t), int ncodes)
{
    if (a >= dec((uint8_t)(ncodes - 1)))
        return ncodes - 1;
    int hi = 0;
    while (dec((uint8_t)hi) < a)
        ++hi;                                   /* first grid value >= a */
    if (hi == 0)
        return 0;
    const double dhi = dec((uint8_t)hi) - a, dlo = a - dec((uint8_t)(hi - 1));
    if (dhi < dlo)
        return hi;
    if (dlo < dhi)
        return hi - 1;
    return (hi % 2 == 0) ? hi : hi - 1;         /* tie: the even code */
}

/* e4m3fn code of y: magnitude codes 0..126 (0x7F is NaN), sign in bit 7. */
uint8_t orc_enc_e4m3(double y)
{
    return (uint8_t)((signbit(y) ? 0x80 : 0) | enc_nearest(fabs(y), orc_dec_e4m3, 127));
}

/* e2m1 code of y: magnitude codes 0..7, sign in bit 3. */
uint8_t orc_enc_e2m1(double y)
{
    return (uint8_t)((signbit(y) ? 0x8 : 0) | enc_nearest(fabs(y), orc_dec_e2m1, 8));
}

/* Per-token e4m3 quantiser.  X [M,K] bf16 bits (row stride ldx elements) ->
 * Q [M,K] e4m3 codes (row stride ldq bytes) and scale [M] binary32. */
void orc_quant_f8_pertoken(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *scale,
                           int64_t M, int64_t K)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *x = X + m * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf(orc_bf16_to_f32(x[k]));
            if (v > amax)
                amax = v;
        }
        const float s = amax / 448.0f;          /* binary32 division */
        scale[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            const float v = orc_bf16_to_f32(x[k]);
            const float y = (s > 0.0f) ? v / s : v; /* s == 0: every v is +-0 */
            Q[m * ldq + k] = orc_enc_e4m3((double)y);
        }
    }
}

/* Blockscale e4m3 quantiser, the operand of orc_f8_blockscale's A: the
 * per-token rule applied to each 128-element block of a row (the blockscale
 * GEMM's block reading): scale S[m, b] = fp32(amax_block / 448) and
 * code = enc(fp32(x / S[m, b])), an all-zero block keeping its signed zeros
 * with scale 0.  X [M,K] bf16 bits (row stride ldx), K % 128 == 0; Q [M,K]
 * codes (row stride ldq bytes); S [M, K/128] binary32 (row stride lds
 * elements).  Returns 0, or -1 if K is not a multiple of 128. */
int orc_quant_f8_block(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *S, int64_t lds,
                       int64_t M, int64_t K)
{
    if (K % 128 != 0)
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < K / 128; ++b) {
            const uint16_t *x = X + m * ldx + 128 * b;
            float amax = 0.0f;
            for (int j = 0; j < 128; ++j) {
                const float v = fabsf(orc_bf16_to_f32(x[j]));
                if (v > amax)
                    amax = v;
            }
            const float s = amax / 448.0f;          /* binary32 division */
            S[m * lds + b] = s;
            for (int j = 0; j < 128; ++j) {
                const float v = orc_bf16_to_f32(x[j]);
                const float y = (s > 0.0f) ? v / s : v;
                Q[m * ldq + 128 * b + j] = orc_enc_e4m3((double)y);
            }
        }
    }
    return 0;
}

/* MX quantiser, one ue8m0 scale per 32 elements of a row.  fmt 0: e4m3, Q
 * [M,K] bytes; fmt 1: e2m1, Q [M,K/2] bytes (element k even in the low nibble
 * of byte k/2, k odd in the high one).  X [M,K] bf16 bits (row stride ldx
 * elements), K % 32 == 0; Q row stride ldq bytes; S [M,K/32] codes, row
 * stride lds bytes.  Returns 0, or -1 for an unknown fmt. */
int orc_quant_mx(int fmt, const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, uint8_t *S,
                 int64_t lds, int64_t M, int64_t K)
{
    if (fmt != 0 && fmt != 1)
        return -1;
    const int emax = (fmt == 0) ? 8 : 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const uint16_t *x = X + m * ldx + 32 * b;
            double amax = 0.0;
            for (int j = 0; j < 32; ++j)
                amax = fmax(amax, fabs((double)orc_bf16_to_f32(x[j])));
            int code = 0;
            if (amax > 0.0) {
                int e;
                frexp(amax, &e);                 /* amax = f * 2^e, f in [0.5, 1) */
                const int X_ = (e - 1) - emax;   /* floor(log2(amax)) - emax */
                code = X_ + 127 < 0 ? 0 : (X_ + 127 > 254 ? 254 : X_ + 127);
            }
            S[m * lds + b] = (uint8_t)code;
            for (int j = 0; j < 32; ++j) {
                const double y = ldexp((double)orc_bf16_to_f32(x[j]), 127 - code);  /* exact */
                if (fmt == 0) {
                    Q[m * ldq + 32 * b + j] = orc_enc_e4m3(y);
                } else {
                    uint8_t *byte = &Q[m * ldq + 16 * b + j / 2];
                    const uint8_t c = orc_enc_e2m1(y);
                    *byte = (j % 2 == 0) ? (uint8_t)((*byte & 0xF0) | c) : (uint8_t)((*byte & 0x0F) | (c << 4));
                }
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------- prepacked B */

/* The weight layout the prepacked GEMM entry points read.  Both MI355X GEMMs
 * on the pages take B in a layout prepared once ("gemm_a8w8_bpreshuffle" in
 * ROCm/aiter PR #6262, description; the "BpreShuffle" FP4 kernel compared
 * against in ROCm/FlyDSL PR #990, description); their orders are their own
 * kernels'.  This library's order: B (N rows of row_bytes bytes, row_bytes a
 * multiple of 64) becomes ceil(N/16) groups of 16 rows; group R is
 * nst = row_bytes/64 blocks of 1024 bytes, block t holding bytes
 * 64t .. 64t+63 of rows 16R .. 16R+15: its 16-byte slot p (0..63) is row
 * 16R + p/4, bytes 64t + 16c .. 64t + 16c + 15 with c = (p mod 4) XOR
 * ((p / 16) mod 4).  Rows at or past N are zeros.
 * Bp[((R*nst + t)*64 + p)*16 + b] = B[16R + p/4][64t + 16c + b]. */
void orc_pack_b(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp)
{
    const int64_t nst = row_bytes / 64, groups = (N + 15) / 16;
    for (int64_t R = 0; R < groups; ++R)
        for (int64_t t = 0; t < nst; ++t)
            for (int p = 0; p < 64; ++p) {
                const int64_t row = 16 * R + p / 4;
                const int c = (p % 4) ^ ((p / 16) % 4);
                uint8_t *dst = Bp + ((R * nst + t) * 64 + p) * 16;
                for (int b = 0; b < 16; ++b)
                    dst[b] = row < N ? B[row * ldb + 64 * t + 16 * c + b] : 0;
            }
}

/* The prepacked layout of an e2m1 B under e4m3 A (the mixed MX GEMM, whose
 * LDS-fetch stages hold 32-byte B rows): ceil(N/32) groups of 32 rows; group
 * R is row_bytes/32 blocks of 1 KB; block t holds bytes 32t .. 32t + 31 of rows
 * 32R .. 32R + 31, its 16-byte slot p being row 32R + p/2, bytes 32t + 16c ..
 * 32t + 16c + 15 with c = (p mod 2) XOR ((p / 16) mod 2).  Rows at or past N
 * are zeros.  row_bytes % 32 == 0.
 * Bp[((R*nst + t)*64 + p)*16 + b] = B[32R + p/2][32t + 16c + b]. */
void orc_pack_b32(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp)
{
    const int64_t nst = row_bytes / 32, groups = (N + 31) / 32;
    for (int64_t R = 0; R < groups; ++R)
        for (int64_t t = 0; t < nst; ++t)
            for (int p = 0; p < 64; ++p) {
                const int64_t row = 32 * R + p / 2;
                const int c = (p % 2) ^ ((p / 16) % 2);
                uint8_t *dst = Bp + ((R * nst + t) * 64 + p) * 16;
                for (int b = 0; b < 16; ++b)
                    dst[b] = row < N ? B[row * ldb + 32 * t + 16 * c + b] : 0;
            }
}

/* ------------------------------------------------- array forms for tests */

void orc_enc_e4m3_array(const double *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_enc_e4m3(in[i]);
}

void orc_enc_e2m1_array(const double *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_enc_e2m1(in[i]);
}


void orc_dec_e4m3_array(const uint8_t *codes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_dec_e4m3(codes[i]);
}

void orc_dec_e2m1_array(const uint8_t *nibbles, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_dec_e2m1(nibbles[i]);
}

void orc_dec_e2m3_array(const uint8_t *codes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_dec_e2m3(codes[i]);
}

void orc_dec_e3m2_array(const uint8_t *codes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_dec_e3m2(codes[i]);
}

/* Element codes of an MX operand row (mx_code), for the tests' packing pins. */
void orc_mx_codes(int fmt, const uint8_t *row, int64_t K, uint8_t *out)
{
    for (int64_t k = 0; k < K; ++k)
        out[k] = (uint8_t)mx_code(row, k, fmt);
}

void orc_dec_ue8m0_array(const uint8_t *codes, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_dec_ue8m0(codes[i]);
}

void orc_bf16_rne_array(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_bf16_rne(in[i]);
}
