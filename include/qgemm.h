/*
 * qgemm.h -- C ABI of the MI355X (gfx950) scaled low-precision GEMM library
 *
 *     C = bf16( scale_A (.) scale_B (.) (A . B^T) + bias )
 *
 * in these element paths:
 *   qgemm_i8_rowwise   int8 A and B, int32 accumulation, fp32 per-row scale of
 *                      A and per-row scale of B ("rowwise"), optional bf16
 *                      bias, bf16 out.  Defined by comfy-kitchen PR #174
 *                      "Optimize HIP WMMA INT8 GEMM staging, epilogue, and
 *                      deep-K tiling": Summary (rowwise scales and bias,
 *                      no-bias signed zero), Validation (exact int8 results),
 *                      Update "rebased onto v0.2.40" (epilogue association
 *                      (acc*sa)*sb).
 *   qgemm_f8_pertoken  e4m3 A and B with fp32 per-token (row of A) and
 *                      per-channel (row of B) scales, the "ptpc" GEMM of
 *                      ROCm/mori PR #806 "perf(gemm-ar): mxfp8 with row-major
 *                      scales staged through LDS", commit message table.
 *   qgemm_f8_blockscale  e4m3 A and B with fp32 scales per 128-element K
 *                      block (A per row, B per 128 rows): the "blockscale"
 *                      GEMM of the same page.
 *   qgemm_mx           MX: e4m3 or e2m1 elements with one ue8m0 scale per 32
 *                      elements along K; A scales [M, K/32] and B scales
 *                      [N/32, K/32] as uint8 row-major ("mxfp8_raw", ROCm/mori
 *                      PR #806, What) or [N, K/32] (the 1x32 FP4 scales of
 *                      ROCm/FlyDSL PR #990 "[fp4_gemm_4wave] MXFP4 GEMM perf
 *                      optimize").
 *   qgemm_mx_mixed     MX with e4m3 A (activations) and e2m1 B (weights),
 *                      or e2m1 A with e4m3 B, each operand under its own
 *                      format and the same ue8m0 per-32 scale rule.
 *
 * Prepacked variants of each GEMM take a B already laid out in the order the
 * kernels' LDS stages use (qgemm_prepack_b, qgemm_prepack_b32).
 *
 * Numerics (all paths): the product is accumulated exactly (int32) for int8
 * and in fp32 by the matrix cores for e4m3 / e2m1; the epilogue is, per
 * output, in binary32 with round-to-nearest-even and no fused operations:
 *     f = (float)acc;  f = f * scale_a[m];  f = f * scale_b[n];   (int8, fp8)
 *     if (bias) f = f + bias[n];
 *     C[m,n] = bf16_round_nearest_even(f)
 * Without bias nothing is added, so a negative-zero product stays -0.
 *
 * Conventions shared by every entry point:
 *  - Every pointer is device memory of the current HIP device, owned by the
 *    caller.  The library keeps no pointer after the call returns and
 *    allocates no device memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    device's default stream).  The call returns once the kernel is queued.
 *  - Arguments are validated on the host before anything is enqueued: on any
 *    non-OK status nothing has been launched and C is untouched.  The text of
 *    the last failure on the calling thread is qgemm_last_error().
 *  - M == 0 or N == 0 is a no-op that returns QGEMM_OK once M, N and K pass
 *    the shape checks (pointers may then be NULL).  K must be a positive
 *    multiple of 32 (the MX block size) and at most 131071 for int8 (the
 *    int32 accumulator cannot overflow below that).
 *  - Only C[0..M) x [0..N) is written; the rest of each ldc-long row is left
 *    alone.  C must not alias any input.
 *  - Alignment: A, B, C 16-byte aligned; lda, ldb (bytes) multiples of 16 and
 *    at least the bytes of one row; ldc (elements) a multiple of 8 and >= N;
 *    scale_a / scale_b (fp32) 4-byte aligned; bias 2-byte aligned; MX scale
 *    arrays have no alignment requirement.  256 * lda and 256 * ldb must stay
 *    below 2^31 bytes.
 *  - The device must be gfx950; anything else returns
 *    QGEMM_ERR_UNSUPPORTED_DEVICE.  There is no fallback path.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QGEMM_OK = 0,
    QGEMM_ERR_NULL_POINTER = 1,       /* a required pointer is NULL (bias may be)      */
    QGEMM_ERR_BAD_SHAPE = 2,          /* M<0, N<0, K<=0, K%32, int8 K>131071, M or N
                                         >= 2^31                                       */
    QGEMM_ERR_BAD_LAYOUT = 3,         /* stride below the row, stride or pointer
                                         misaligned, 256*ld beyond 2^31 bytes         */
    QGEMM_ERR_BAD_FORMAT = 4,         /* unknown MX element format or B-scale layout  */
    QGEMM_ERR_UNSUPPORTED_DEVICE = 5, /* current device is not gfx950                 */
    QGEMM_ERR_HIP = 6                 /* HIP reported an error; see qgemm_last_error  */
} qgemm_status;

/* MX element format, the same for A and B.  The pages name the MX GEMM with
 * e4m3 and e2m1 elements; E2M3 and E3M2 are the 6-bit (FP6) element types OCP
 * Microscaling v1.0 defines beside them, under the same block rule. */
typedef enum {
    QGEMM_MX_E4M3 = 0, /* OCP E4M3FN, one byte per element                          */
    QGEMM_MX_E2M1 = 1, /* OCP E2M1, two per byte: element k (k even) in bits 3:0 of
                          byte k/2, element k+1 in bits 7:4                         */
    QGEMM_MX_E2M3 = 2, /* OCP FP6 E2M3 (max 7.5), four per three bytes: element k in
                          bits 6k..6k+5 of the row, bit b of a row being bit b%8 of
                          byte b/8 (lowest bits first); rows of 3K/4 bytes         */
    QGEMM_MX_E3M2 = 3  /* OCP FP6 E3M2 (max 28), packed as E2M3                     */
} qgemm_mx_fmt;

/* Rows of B that share one ue8m0 scale per 32-element K block. */
typedef enum {
    QGEMM_MX_BSCALE_1x32 = 1,  /* scale_b is [N, K/32]            */
    QGEMM_MX_BSCALE_32x32 = 32 /* scale_b is [ceil(N/32), K/32]   */
} qgemm_mx_bscale;

/* INT8 rowwise GEMM.
 *   A        [M, K] int8, row stride lda bytes
 *   B        [N, K] int8, row stride ldb bytes
 *   scale_a  [M] fp32, scale_b [N] fp32 (any finite values, sign kept)
 *   bias     [N] bf16 bit patterns, or NULL for no bias
 *   C        [M, ldc] bf16 bit patterns (output)
 * acc[m,n] = sum_k A[m,k]*B[n,k] in int32, exact; then the epilogue above. */
qgemm_status qgemm_i8_rowwise(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                              const float *scale_a, const float *scale_b, const uint16_t *bias,
                              uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              void *stream);

/* The INT8 product alone: C[m,n] = sum_k A[m,k]*B[n,k] as int32 (the
 * accumulator qgemm_i8_rowwise applies its epilogue to), C [M, ldc] int32.
 * Same operand conventions as qgemm_i8_rowwise. */
qgemm_status qgemm_i8_acc_i32(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                              int32_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              void *stream);

/* FP8 e4m3 per-token / per-channel GEMM.
 *   A        [M, K] e4m3fn codes, row stride lda bytes
 *   B        [N, K] e4m3fn codes, row stride ldb bytes
 *   scale_a  [M] fp32 per token, scale_b [N] fp32 per channel
 *   bias, C  as for qgemm_i8_rowwise
 * acc[m,n] = sum_k e4m3(A[m,k]) * e4m3(B[n,k]) in fp32 (matrix cores); then
 * the epilogue above.  NaN codes propagate. */
qgemm_status qgemm_f8_pertoken(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                               const float *scale_a, const float *scale_b, const uint16_t *bias,
                               uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               void *stream);

/* FP8 e4m3 GEMM with block-wise fp32 scales, the "blockscale" GEMM that
 * ROCm/mori PR #806 "perf(gemm-ar): mxfp8 with row-major scales staged
 * through LDS" measures next to "ptpc" and "mxfp8" (commit message table).
 * The page names no block sizes; this entry point takes K blocks of 128:
 *   A        [M, K] e4m3fn codes, row stride lda bytes
 *   B        [N, K] e4m3fn codes, row stride ldb bytes
 *   scale_a  fp32 [M, K/128], row-major, row stride K/128: one scale per row
 *            of A and K block (per token)
 *   scale_b  fp32 [ceil(N/128), K/128], row-major: one scale per 128 rows of
 *            B and K block
 *   bias, C  as for qgemm_i8_rowwise
 * acc = sum_kb scale_a[m,kb] * scale_b[n/128,kb] * P[kb], P[kb] the fp32
 * matrix-core sum of the block's 128 products, each block folded into the
 * fp32 total with one fused multiply-add; then f = acc, [+ bias], bf16
 * round-nearest-even.  K must be a multiple of 128 (QGEMM_ERR_BAD_SHAPE) and
 * both scale arrays 8-byte aligned (QGEMM_ERR_BAD_LAYOUT). */
qgemm_status qgemm_f8_blockscale(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                 const float *scale_a, const float *scale_b, const uint16_t *bias,
                                 uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                 void *stream);

/* MX GEMM (block-scaled e4m3, e2m1, or the 6-bit e2m3 / e3m2).
 *   A        [M, K] elements of fmt, row stride lda_bytes (K, K/2 or 3K/4 bytes
 *            of data)
 *   B        [N, K] elements of fmt, row stride ldb_bytes
 *   scale_a  ue8m0 [M, K/32], row-major, row stride K/32 bytes
 *   scale_b  ue8m0 [N, K/32] (b_layout 1x32) or [ceil(N/32), K/32] (32x32)
 *   bias, C  as for qgemm_i8_rowwise
 * A~[m,k] = fmt(A[m,k]) * 2^(scale_a[m,k/32]-127), B~ likewise with the scale
 * of row n (1x32) or n/32 (32x32); acc = sum_k A~ B~ in fp32 (matrix cores);
 * then f = acc, [+ bias], bf16 round-nearest-even.  Scale code 255 is NaN.
 * The 6-bit formats need K a multiple of 128 (QGEMM_ERR_BAD_SHAPE) and 8-byte
 * aligned scale arrays (QGEMM_ERR_BAD_LAYOUT); qgemm_mx_prepacked does not take
 * them (QGEMM_ERR_BAD_FORMAT).  e4m3 and e2m1 take any K a multiple of 32,
 * and run the LDS-fetch tiles with 8-byte aligned scale arrays: e4m3 at any
 * such K, e2m1 where K % 128 == 0 and, in stages of 64 elements (tiles 4, 5,
 * 7; M > 16), at the other K; otherwise the register-staged tile. */
qgemm_status qgemm_mx(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *B,
                      int64_t ldb_bytes, const uint8_t *scale_a, const uint8_t *scale_b,
                      qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc,
                      int64_t M, int64_t N, int64_t K, void *stream);

/* MX GEMM with a format per operand: fmt_a for A, fmt_b for B, otherwise as
 * qgemm_mx (one ue8m0 scale per 32 elements along K for each operand, the
 * scale layouts of qgemm_mx).  Equal formats are qgemm_mx.  Both mixed pairs
 * of e4m3 and e2m1 are supported:
 *   e4m3 A (activations), e2m1 B (weights):
 *     A      [M, K] e4m3fn codes, row stride lda_bytes (>= K)
 *     B      [N, K] e2m1, two per byte (even k in the low nibble), row stride
 *            ldb_bytes (>= K/2)
 *   e2m1 A, e4m3 B: the same with the operands' formats swapped (lda_bytes
 *            >= K/2, ldb_bytes >= K); every M runs an LDS-fetch tile (4, 5
 *            or 7; no small-M form).
 * Either needs K a multiple of 32 (QGEMM_ERR_BAD_SHAPE) and 8-byte aligned
 * scale arrays (QGEMM_ERR_BAD_LAYOUT).  Numerics as qgemm_mx. */
qgemm_status qgemm_mx_mixed(qgemm_mx_fmt fmt_a, qgemm_mx_fmt fmt_b, const void *A, int64_t lda_bytes,
                            const void *B, int64_t ldb_bytes, const uint8_t *scale_a, const uint8_t *scale_b,
                            qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc,
                            int64_t M, int64_t N, int64_t K, void *stream);

/* The mixed GEMM (e4m3 A, e2m1 B) on a prepacked B.  qgemm_prepack_b32
 * rewrites B [N, row_bytes] (row_bytes = K/2, a positive multiple of 128;
 * row stride ldb bytes, 16-byte aligned, ldb a multiple of 16) into Bp
 * (qgemm_prepacked_b32_bytes(N, row_bytes) bytes, 16-byte aligned,
 * caller-owned): ceil(N/32) groups of 32 rows, group R holding row_bytes/32
 * blocks of 1 KB, block t bytes 32t .. 32t+31 of the group's rows, 16-byte
 * slot p being row 32R + p/2, chunk (p mod 2) XOR ((p/16) mod 2); rows past N
 * are zeros -- the order the mixed GEMM's B stages take in LDS.
 * qgemm_prepacked_b32_bytes returns -1 for a bad size.  qgemm_mx_mixed_prepacked
 * is qgemm_mx_mixed with Bp in place of (B, ldb) and K a multiple of 256 (the
 * packer's rows): for e4m3 A, Bp is an e2m1 B [N, K/2] packed by
 * qgemm_prepack_b32 (M <= 16 runs the 128x128 tile); for e2m1 A, an e4m3 B
 * [N, K] packed by qgemm_prepack_b (qgemm_prepack_b's layout, below).  Equal
 * formats return QGEMM_ERR_BAD_FORMAT.  Results equal qgemm_mx_mixed's on the
 * same tile. */
int64_t qgemm_prepacked_b32_bytes(int64_t N, int64_t row_bytes);
qgemm_status qgemm_prepack_b32(const void *B, int64_t ldb, int64_t N, int64_t row_bytes, void *Bp, void *stream);
qgemm_status qgemm_mx_mixed_prepacked(qgemm_mx_fmt fmt_a, qgemm_mx_fmt fmt_b, const void *A, int64_t lda_bytes,
                                      const void *Bp, const uint8_t *scale_a, const uint8_t *scale_b,
                                      qgemm_mx_bscale b_layout, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                      int64_t M, int64_t N, int64_t K, void *stream);

/* Prepacked B.  B (the weights, static across calls) can be rewritten once
 * into the order the LDS-fetch kernel's B stages take in LDS, so that each
 * of its fetches reads one contiguous kilobyte instead of 16 rows x 64 bytes
 * (on one MI355X: INT8 30000x21504x5376 +4.5%, MXFP4 8192^3 +6%, MXFP8
 * 16384x7168x2048 +3%, FP8 4096x2112x7168 +11%).  The MI355X
 * GEMMs on the pages read such a prepared B too ("gemm_a8w8_bpreshuffle",
 * ROCm/aiter PR #6262, description; the "BpreShuffle" FP4 kernel of
 * ROCm/FlyDSL PR #990, description); the order here is this library's own:
 *   ceil(N/16) groups of 16 rows; group R is row_bytes/64 blocks of 1024
 *   bytes; block t holds bytes 64t .. 64t+63 of rows 16R .. 16R+15, its
 *   16-byte slot p (0..63) being row 16R + p/4, bytes 64t + 16c .. +15,
 *   c = (p mod 4) XOR ((p/16) mod 4); rows at or past N are zeros.
 * row_bytes = K (int8, e4m3) or K/2 (e2m1), a positive multiple of 256 with
 * 256 * row_bytes below 2^31.  The layout does not depend on the element type
 * or the scales. */

/* Bytes of a prepacked B: ceil(N/16) * 16 * row_bytes, or -1 if N or
 * row_bytes is out of range.  Pure host logic. */
int64_t qgemm_prepacked_b_bytes(int64_t N, int64_t row_bytes);

/* Write B [N, row_bytes] (row stride ldb bytes, 16-byte aligned, ldb a
 * multiple of 16) into Bp (qgemm_prepacked_b_bytes(N, row_bytes) bytes,
 * 16-byte aligned, caller-owned, not overlapping B).  Asynchronous on stream;
 * N == 0 is a no-op. */
qgemm_status qgemm_prepack_b(const void *B, int64_t ldb, int64_t N, int64_t row_bytes, void *Bp, void *stream);

/* The three GEMMs with B prepacked by qgemm_prepack_b (row_bytes = the row of
 * B the call would otherwise take).  Same arguments, numerics and results as
 * qgemm_i8_rowwise / qgemm_f8_pertoken / qgemm_mx with Bp in place of (B,
 * ldb); in addition K must give rows of a multiple of 256 bytes
 * (QGEMM_ERR_BAD_SHAPE otherwise) and, for MX, K/32 must be a multiple of 16
 * (e2m1) or 8 (e4m3) with scale arrays aligned to 16 (e2m1) or 8 (e4m3) bytes
 * (QGEMM_ERR_BAD_LAYOUT otherwise).  INT8
 * results are bit-identical to qgemm_i8_rowwise's; FP8 / MX results equal
 * those of qgemm_*'s LDS-fetch tiles. */
qgemm_status qgemm_i8_rowwise_prepacked(const int8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                        const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                        int64_t M, int64_t N, int64_t K, void *stream);
qgemm_status qgemm_f8_pertoken_prepacked(const uint8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                         const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                         int64_t M, int64_t N, int64_t K, void *stream);
/* qgemm_f8_blockscale with Bp in place of (B, ldb) and K a multiple of 256
 * (the packer's rows): results equal qgemm_f8_blockscale's on the same tile. */
qgemm_status qgemm_f8_blockscale_prepacked(const uint8_t *A, int64_t lda, const void *Bp, const float *scale_a,
                                           const float *scale_b, const uint16_t *bias, uint16_t *C, int64_t ldc,
                                           int64_t M, int64_t N, int64_t K, void *stream);
qgemm_status qgemm_mx_prepacked(qgemm_mx_fmt fmt, const void *A, int64_t lda_bytes, const void *Bp,
                                const uint8_t *scale_a, const uint8_t *scale_b, qgemm_mx_bscale b_layout,
                                const uint16_t *bias, uint16_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                void *stream);

/* Per-token e4m3 quantiser: the A operand and scale_a of qgemm_f8_pertoken
 * from bf16 activations.  "perf(gemm-ar): mxfp8 with row-major scales staged
 * through LDS" (ROCm/mori PR #806), Measured, names the per-token ("ptpc")
 * scales; the page gives no formula, and the one taken is:
 *   scale[m] = fp32( amax_m / 448 ),  amax_m = max_k |X[m,k]|  (binary32)
 *   Q[m,k]   = enc_e4m3( fp32( X[m,k] / scale[m] ) )          (IEEE division)
 * enc: the nearest e4m3fn value, ties to the even code, magnitudes beyond 448
 * saturating to 448, the sign bit copied from the value (a negative value
 * that rounds to zero gives -0, 0x80).  A row of zeros gets scale 0 and each
 * zero's own sign.
 *   X      [M, K] bf16 bit patterns, row stride ldx ELEMENTS (multiple of 8)
 *   Q      [M, K] e4m3fn codes (output), row stride ldq bytes (multiple of 16)
 *   scale  [M] fp32 (output), 4-byte aligned
 * X and Q 16-byte aligned; K a positive multiple of 32; Q and scale must not
 * overlap X.  Inputs are finite: a row holding NaN or infinity gets
 * unspecified codes and scale.  Nothing outside Q's [M, K] and scale[0..M)
 * is written. */
qgemm_status qgemm_quant_f8_pertoken(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *scale,
                                     int64_t M, int64_t K, void *stream);

/* MX quantiser: the A operand and scale_a of qgemm_mx from bf16 activations,
 * one ue8m0 scale per 32 elements of a row, handed over as [M, K/32] uint8
 * row-major as ROCm/mori PR #806 ("perf(gemm-ar): mxfp8 with row-major scales
 * staged through LDS", What) describes the quantiser's output.  The scale
 * rule is the OCP Microscaling v1.0 one:
 *   X_b   = floor(log2(amax_b)) - emax   (emax 8 for e4m3, 2 for e2m1)
 *   S     = X_b + 127 clamped to [0, 254]; 0 for an all-zero block
 *   code  = enc( X[m,k] * 2^-(S - 127) )  (exact scaling by a power of two)
 * enc as for qgemm_quant_f8_pertoken, on the e4m3fn grid (max 448) or the
 * e2m1 grid (max 6).
 *   fmt    QGEMM_MX_E4M3: Q [M, K] bytes; QGEMM_MX_E2M1: Q [M, K/2] bytes,
 *          element k (k even) in bits 3:0 of byte k/2, k+1 in bits 7:4
 *   X      [M, K] bf16 bit patterns, row stride ldx ELEMENTS (multiple of 8)
 *   Q      row stride ldq bytes (multiple of 16)
 *   S      [M, K/32] ue8m0 codes (output), row stride lds bytes (>= K/32)
 * X and Q 16-byte aligned; K a positive multiple of 32; outputs must not
 * overlap X.  Inputs are finite: a block holding NaN or infinity gets
 * unspecified codes and scale.  Nothing outside Q's [M, K] elements and S's
 * [M, K/32] is written. */
qgemm_status qgemm_quant_mx(qgemm_mx_fmt fmt, const uint16_t *X, int64_t ldx, void *Q, int64_t ldq, uint8_t *S,
                            int64_t lds, int64_t M, int64_t K, void *stream);

/* Blockscale e4m3 quantiser: bf16 activations -> the A operand and A scales
 * of qgemm_f8_blockscale (the per-token rule applied to each 128-element
 * block of a row; the page names the blockscale GEMM, the block reading is
 * the library's).
 *   X      [M, K] bf16 bits, row stride ldx elements (multiple of 8)
 *   Q      [M, K] e4m3fn codes (output), row stride ldq bytes (multiple of 16)
 *   S      [M, K/128] fp32 scales (output), row stride lds elements (>= K/128)
 * Per row m and block b: S[m,b] = fp32(amax / 448) over the block's |x|,
 * Q = e4m3(fp32(x / S[m,b])) (nearest, ties to even, saturating, sign kept;
 * an all-zero block gets scale 0 and keeps its signed zeros).  K must be a
 * multiple of 128 (QGEMM_ERR_BAD_SHAPE); X and Q 16-byte aligned, S 4-byte
 * aligned; outputs must not overlap X. */
qgemm_status qgemm_quant_f8_block(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *S, int64_t lds,
                                  int64_t M, int64_t K, void *stream);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char *qgemm_last_error(void);

/* Fixed name of a status code, e.g. "QGEMM_ERR_BAD_SHAPE". */
const char *qgemm_status_string(qgemm_status status);

/* Tile variant the host-side table picks for a problem (pure host logic, no
 * HIP call; for MX, assuming 16-byte-aligned scale arrays).  path: 0 int8,
 * 1 fp8, 2 MX e4m3, 3 MX e2m1 (at K % 128 != 0 and M > 16: tile 5 where
 * the table picks 256x256, else 7), 4 fp8 blockscale (tile 8 for M <= 16, else
 * tile 10 when its grid of 256x128 tiles fills the 256 CUs at least once,
 * else tile 7), 5 MX e4m3 A with e2m1 B (tile 8 for M <= 16, else tile 4
 * where the table picks 256x256, else 7), 6 / 7 MX with 6-bit E2M3 / E3M2
 * elements (tile 4 where the table picks 256x256, else 7; no small-M tile),
 * 8 MX e2m1 A with e4m3 B (as 6 / 7).
 * Returns the tile id, or -1 for a bad path:
 *   0: 256x256, 4 waves, operands staged through registers
 *   1: 128x128    2: 256x256 with 8 waves, staged through registers
 *   3: 192x192
 *   4: 256x256, 4 waves, operands fetched straight into LDS
 *   5: 256x256, 8 waves, operands fetched straight into LDS
 *   6: 192x192, 4 waves, operands fetched straight into LDS
 *   7: 128x128, 4 waves, operands fetched straight into LDS
 *   8: 16 rows x 16 columns, 8 waves splitting K (small M)
 *   9: 64 rows x 16 columns, 8 waves splitting K (small M)
 *  10: 256 rows x 128 columns, fp8 blockscale only
 * Tiles 4-7 need K bytes a multiple of 64 (whole stages; a last round of
 * fewer than four is masked) and, for e2m1 MX, K % 128 (e4m3 MX and the mixed
 * pairs: any K % 32, e2m1 at K % 128 != 0 as above), with scale arrays
 * aligned to 16 (e2m1) or 8 (e4m3) bytes; where these hold, the table's 256x256 choice runs as tile 4 (mixed and 6-bit MX, and
 * INT8 on a prepacked B) or 5 (the others), 192x192 as tile 6 and 128x128 as tile 7.  Calls with M <= 64 take tile 8
 * (M <= 16) or 9 (INT8 and FP8 only: MX takes the small-M kernel up to
 * M = 16). */
int qgemm_select_tile(int path, int64_t M, int64_t N, int64_t K);

/* Rows of A one tile covers (for tiles 0-7 also the rows of B; tiles 8 and 9
 * cover 16 rows of B, tile 10 128), or 0 for an unknown id. */
int qgemm_tile_rows(int tile);

/* Force a tile id for later calls on the calling thread (benchmarks and the
 * variant-equivalence tests); -1 restores the table.  Returns the previous
 * value, or -2 (and changes nothing) for an unknown id.  A forced LDS-fetch
 * tile whose requirements a call does not meet runs as tile 0. */
int qgemm_force_tile(int tile);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
