// qgemm_quant.hip -- activation quantisers: bf16 activations -> the A operand
// and A scales of the FP8 per-token GEMM and of the MX GEMM.
//
// "perf(gemm-ar): mxfp8 with row-major scales staged through LDS" (ROCm/mori
// PR #806), What: the quantiser hands the GEMM A's ue8m0 scales as [M, K/32]
// uint8, row-major -- the layout qgemm_mx reads.  Measured: per-token
// ("ptpc") FP8 scales, one fp32 per row of A.  The scale rules (per-token
// amax/448; the OCP Microscaling shared exponent floor(log2 amax) - emax) and
// the element rounding (nearest, ties to even, saturating, sign kept) are
// the readings the library documents with these entry points.
//
// Both kernels move bytes and do a little ALU work per element: HBM-bound,
// no matrix cores.
//  * Per-token: one workgroup of 256 threads per row.  A thread keeps up to
//    4 of the row's 16-byte pieces in registers (rows up to 8192 elements
//    are read once); the row's max |x| comes from butterfly shuffles within
//    each wave and the four wave maxima in LDS; then each thread divides and
//    rounds from its registers, re-reading (from L2) pieces beyond the 4.
//    The division is the IEEE binary32 one (the compiler's correctly rounded
//    sequence), as the definition fixes the quotient.
//  * MX: four lanes per 32-element block, 8 elements (one 16-byte load) per
//    lane and four such blocks per thread, all loaded first; the block's max
//    |x| by two shuffles; the scale code comes from the
//    max's binary32 exponent field E: floor(log2 amax) = E - 127 for a normal
//    amax, and a subnormal or zero amax gives code 0 either way, so the code
//    is max(E - emax, 0).  Scaling by 2^(127 - code) is exact (a power of two,
//    no overflow since |x| <= amax < 2^(E - 126)).
//  * Blockscale e4m3 (one fp32 scale per 128 elements of a row, the operand of
//    the blockscale GEMM): sixteen lanes per block, one 16-byte load each and
//    four blocks per thread loaded first; the block max by four shuffles, then
//    the per-token rule within the block (scale amax/448, IEEE division).
//  * The codes are written with non-temporal stores (whole rows per wave;
//    one MI355X: per-token 4096x7168 +5%, MX e4m3 16384x2048 +10%, e2m1
//    unchanged); non-temporal loads of X were slower.
//  * Rounding to the element grid works on the binary32 bits: for a
//    magnitude in the normal range, adding half an element step minus one
//    plus the kept lowest bit and truncating rounds to nearest even, a carry
//    into the exponent included; below the smallest normal the step is fixed
//    and rintf (round half to even) on the value over the step gives the code.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemm_quant.hpp"

namespace qgemm {

typedef unsigned u32x4q __attribute__((ext_vector_type(4)));
typedef unsigned u32x2q __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// e4m3fn code of y (OCP 8-bit floating point): magnitudes up to 448, step
// 2^(e-3) on [2^e, 2^(e+1)) for e >= -6 and 2^-9 below 2^-6; sign in bit 7.
__device__ __forceinline__ unsigned enc_e4m3(float y)
{
    const unsigned sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    unsigned mag;
    if (a < 0.015625f) {
        mag = (unsigned)__builtin_rintf(a * 512.0f);              // 0..8
    } else {
        const unsigned b = __float_as_uint(a);
        // keep 3 mantissa bits; exponent bias 127 -> 7: (127 - 7) << 3 = 960
        mag = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - 960u;
    }
    return sign | mag;
}

// e2m1 code of y (OCP Microscaling FP4): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
// 6; sign in bit 3.
__device__ __forceinline__ unsigned enc_e2m1(float y)
{
    const unsigned sign = (__float_as_uint(y) >> 28) & 0x8u;
    const float a = fminf(fabsf(y), 6.0f);
    unsigned mag;
    if (a < 1.0f) {
        mag = (unsigned)__builtin_rintf(a * 2.0f);                // 0..2
    } else {
        const unsigned b = __float_as_uint(a);
        // keep 1 mantissa bit; exponent bias 127 -> 1: (127 - 1) << 1 = 252
        mag = ((b + 0x1fffffu + ((b >> 22) & 1u)) >> 22) - 252u;
    }
    return sign | mag;
}

__device__ __forceinline__ float piece_amax(u32x4q w)
{
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
    return m;
}

// ------------------------------------------------------------ per-token e4m3

constexpr int PT_THREADS = 256;   // one workgroup per row
constexpr int PT_KEEP = 4;        // 16-byte pieces a thread keeps in registers

__device__ __forceinline__ u32x2q pertoken_codes(u32x4q w, float s)
{
    unsigned c[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = bf16_lo(w[q]), hi = bf16_hi(w[q]);
        // s == 0 only for a row of zeros: keep each zero (and its sign)
        c[2 * q] = enc_e4m3(s > 0.0f ? lo / s : lo);
        c[2 * q + 1] = enc_e4m3(s > 0.0f ? hi / s : hi);
    }
    return u32x2q{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
}

__global__ void __launch_bounds__(PT_THREADS) quant_f8_pertoken_kernel(const uint16_t *X, int64_t ldx, uint8_t *Q,
                                                                        int64_t ldq, float *scale, int M, int K)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int row = blockIdx.x;
    const u32x4q *x = (const u32x4q *)(X + (int64_t)row * ldx);
    u32x2q *q = (u32x2q *)(Q + (int64_t)row * ldq);
    const int nv = K / 8;

    u32x4q keep[PT_KEEP];
#pragma unroll
    for (int c = 0; c < PT_KEEP; ++c) {
        const int v = t + PT_THREADS * c;
        keep[c] = v < nv ? x[v] : u32x4q{0, 0, 0, 0};
    }
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < PT_KEEP; ++c)
        amax = fmaxf(amax, piece_amax(keep[c]));
    for (int v = t + PT_THREADS * PT_KEEP; v < nv; v += PT_THREADS)
        amax = fmaxf(amax, piece_amax(x[v]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float wmax[PT_THREADS / 64];
    if (lane == 0)
        wmax[wave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < PT_THREADS / 64; ++w)
        amax = fmaxf(amax, wmax[w]);

    const float s = amax / 448.0f;
    if (t == 0)
        scale[row] = s;
#pragma unroll
    for (int c = 0; c < PT_KEEP; ++c) {
        const int v = t + PT_THREADS * c;
        if (v < nv)
            __builtin_nontemporal_store(pertoken_codes(keep[c], s), &q[v]);
    }
    for (int v = t + PT_THREADS * PT_KEEP; v < nv; v += PT_THREADS)
        __builtin_nontemporal_store(pertoken_codes(x[v], s), &q[v]);
}

// ------------------------------------------------------------ MX

constexpr int MX_U = 4;   // quarter blocks per thread, loaded before any is used

// Quarter g of the launch (8 elements, one 16-byte load) is quarter g % 4 of
// block g / 4 of the launch's rows: row (g / 4) / kb, block (g / 4) % kb.
// Thread t of workgroup w takes the quarters w * 1024 + t + 256 u, u < 4, so
// a block's four quarters sit on four neighbouring lanes.  The launch covers
// rows * kb * 4 quarters (below 2^31: the host splits larger calls).
template <int FMT>
__global__ void __launch_bounds__(256) quant_mx_kernel(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq,
                                                       uint8_t *S, int64_t lds, unsigned rows, unsigned kb)
{
    constexpr unsigned EMAX = FMT == 0 ? 8u : 2u;
    const unsigned total = rows * kb * 4u;
    const unsigned base = blockIdx.x * (256u * MX_U) + threadIdx.x, part = threadIdx.x & 3u;
    u32x4q w[MX_U];
    unsigned row[MX_U], b[MX_U];
#pragma unroll
    for (int u = 0; u < MX_U; ++u) {
        const unsigned g = base + 256u * u, blk = g >> 2;
        row[u] = blk / kb;
        b[u] = blk - row[u] * kb;
        // a block's four lanes agree on g < total (total is a multiple of 4)
        w[u] = g < total ? *(const u32x4q *)(X + (int64_t)row[u] * ldx + 32 * b[u] + 8 * part)
                         : u32x4q{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < MX_U; ++u) {
        float amax = piece_amax(w[u]);
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        if (base + 256u * u >= total)
            continue;
        const unsigned E = (__float_as_uint(amax) >> 23) & 0xffu;
        const unsigned code = E > EMAX ? E - EMAX : 0u;            // <= 254 - EMAX for finite input
        const float mul = __uint_as_float((254u - code) << 23);    // 2^(127 - code)
        unsigned c[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float lo = bf16_lo(w[u][q]) * mul, hi = bf16_hi(w[u][q]) * mul;
            c[2 * q] = FMT == 0 ? enc_e4m3(lo) : enc_e2m1(lo);
            c[2 * q + 1] = FMT == 0 ? enc_e4m3(hi) : enc_e2m1(hi);
        }
        uint8_t *qrow = Q + (int64_t)row[u] * ldq;
        if constexpr (FMT == 0) {
            const u32x2q v = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                              c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
            __builtin_nontemporal_store(v, (u32x2q *)(qrow + 32 * b[u] + 8 * part));
        } else {
            unsigned v = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v |= c[i] << (4 * i);                            // element 2j low nibble, 2j+1 high
            __builtin_nontemporal_store(v, (unsigned *)(qrow + 16 * b[u] + 4 * part));
        }
        if (part == 0)
            S[(int64_t)row[u] * lds + b[u]] = (uint8_t)code;
    }
}

// ------------------------------------------------------------ blockscale e4m3

// Piece g of the launch (8 elements, one 16-byte load) is piece g % 16 of
// block g / 16 of the launch's rows: row (g / 16) / kb, block (g / 16) % kb.
// Thread t of workgroup w takes the pieces w * 1024 + t + 256 u, u < 4, so a
// block's sixteen pieces sit on sixteen neighbouring lanes (an aligned group).
__global__ void __launch_bounds__(256) quant_f8_block_kernel(const uint16_t *X, int64_t ldx, uint8_t *Q,
                                                             int64_t ldq, float *S, int64_t lds, unsigned rows,
                                                             unsigned kb)
{
    const unsigned total = rows * kb * 16u;
    const unsigned base = blockIdx.x * (256u * MX_U) + threadIdx.x, part = threadIdx.x & 15u;
    u32x4q w[MX_U];
    unsigned row[MX_U], b[MX_U];
#pragma unroll
    for (int u = 0; u < MX_U; ++u) {
        const unsigned g = base + 256u * u, blk = g >> 4;
        row[u] = blk / kb;
        b[u] = blk - row[u] * kb;
        // a block's sixteen lanes agree on g < total (total is a multiple of 16)
        w[u] = g < total ? *(const u32x4q *)(X + (int64_t)row[u] * ldx + 128 * b[u] + 8 * part)
                         : u32x4q{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < MX_U; ++u) {
        float amax = piece_amax(w[u]);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
        if (base + 256u * u >= total)
            continue;
        const float s = amax / 448.0f;
        uint8_t *qrow = Q + (int64_t)row[u] * ldq;
        __builtin_nontemporal_store(pertoken_codes(w[u], s), (u32x2q *)(qrow + 128 * b[u] + 8 * part));
        if (part == 0)
            S[(int64_t)row[u] * lds + b[u]] = s;
    }
}

// ------------------------------------------------------------ launchers

hipError_t launch_quant_f8_pertoken(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *scale,
                                    int M, int K, hipStream_t s)
{
    hipLaunchKernelGGL(quant_f8_pertoken_kernel, dim3((unsigned)M), dim3(PT_THREADS), 0, s, X, ldx, Q, ldq, scale,
                       M, K);
    return hipGetLastError();
}

hipError_t launch_quant_f8_block(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *S, int64_t lds,
                                 int M, int K, hipStream_t s)
{
    const int64_t kb = K / 128;
    // rows per launch: keep rows * kb * 16 pieces (rounded up to whole
    // workgroups) below 2^31
    const int64_t per_wg = 256 * MX_U;
    const int64_t max_rows = (((int64_t)1 << 31) - per_wg) / (16 * kb);
    for (int64_t r0 = 0; r0 < M; r0 += max_rows) {
        const int64_t rows = M - r0 < max_rows ? M - r0 : max_rows;
        const unsigned grid = (unsigned)((rows * kb * 16 + per_wg - 1) / per_wg);
        hipLaunchKernelGGL(quant_f8_block_kernel, dim3(grid), dim3(256), 0, s, X + r0 * ldx, ldx, Q + r0 * ldq, ldq,
                           S + r0 * lds, lds, (unsigned)rows, (unsigned)kb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_quant_mx(int fmt, const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, uint8_t *S,
                           int64_t lds, int M, int K, hipStream_t s)
{
    const int64_t kb = K / 32;
    // rows per launch: keep rows * kb * 4 quarters (rounded up to whole
    // workgroups) below 2^31
    const int64_t per_wg = 256 * MX_U;
    const int64_t max_rows = (((int64_t)1 << 31) - per_wg) / (4 * kb);
    for (int64_t r0 = 0; r0 < M; r0 += max_rows) {
        const int64_t rows = M - r0 < max_rows ? M - r0 : max_rows;
        const unsigned grid = (unsigned)((rows * kb * 4 + per_wg - 1) / per_wg);
        const uint16_t *x = X + r0 * ldx;
        uint8_t *q = Q + r0 * ldq;
        uint8_t *sc = S + r0 * lds;
        if (fmt == 0)
            hipLaunchKernelGGL(quant_mx_kernel<0>, dim3(grid), dim3(256), 0, s, x, ldx, q, ldq, sc, lds,
                               (unsigned)rows, (unsigned)kb);
        else
            hipLaunchKernelGGL(quant_mx_kernel<1>, dim3(grid), dim3(256), 0, s, x, ldx, q, ldq, sc, lds,
                               (unsigned)rows, (unsigned)kb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace qgemm
