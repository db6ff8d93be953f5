// qgemm_pack.hip -- B (the weights, static across calls) rewritten once into
// the order the LDS-fetch kernel's B stages take in LDS, so that its fetches
// read whole kilobytes instead of 16 rows x 64 bytes.
//
// The MI355X GEMMs on the pages read a B prepared ahead of time
// ("gemm_a8w8_bpreshuffle", ROCm/aiter PR #6262, description; the
// "BpreShuffle" FP4 kernel of ROCm/FlyDSL PR #990, description); their orders
// belong to their kernels.  This library's order: ceil(N/16) groups of 16
// rows; group R is row_bytes/64 blocks of 1 KB, block t holding bytes
// 64t .. 64t+63 of rows 16R .. 16R+15, its 16-byte slot p being row 16R + p/4,
// chunk (p mod 4) XOR ((p/16) mod 4) -- exactly the 1 KB one fetch instruction
// of the LDS-fetch kernel writes (lane p to slot p).  Rows past N are zeros.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qgemm_pack.hpp"

namespace qgemm {

typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

// One thread per 16-byte slot of the output: consecutive threads write
// consecutive slots (whole kilobytes per wave), reading 16 rows x 64 bytes.
__global__ void __launch_bounds__(256) prepack_b_kernel(const uint8_t *B, int64_t ldb, int64_t N, int64_t nst,
                                                        uint8_t *Bp, int64_t slots)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= slots)
        return;
    const int p = (int)(o & 63);
    const int64_t blk = o >> 6;                  // block (R, t) = R * nst + t
    const int64_t R = blk / nst, t = blk - R * nst;
    const int64_t row = 16 * R + p / 4;
    const int c = (p & 3) ^ ((p >> 4) & 3);
    u32x4p v = {0, 0, 0, 0};
    if (row < N)
        v = *(const u32x4p *)(B + row * ldb + 64 * t + 16 * c);
    *(u32x4p *)(Bp + 16 * o) = v;
}

// The mixed MX GEMM's e2m1 B (32-byte stage rows): 32-row groups, block t of a
// group holding bytes 32t .. 32t+31 of its rows, slot p being row p/2, chunk
// (p mod 2) XOR ((p/16) mod 2) -- the 1 KB one B fetch of that kernel writes.
__global__ void __launch_bounds__(256) prepack_b32_kernel(const uint8_t *B, int64_t ldb, int64_t N, int64_t nst,
                                                          uint8_t *Bp, int64_t slots)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= slots)
        return;
    const int p = (int)(o & 63);
    const int64_t blk = o >> 6;                  // block (R, t) = R * nst + t
    const int64_t R = blk / nst, t = blk - R * nst;
    const int64_t row = 32 * R + p / 2;
    const int c = (p & 1) ^ ((p >> 4) & 1);
    u32x4p v = {0, 0, 0, 0};
    if (row < N)
        v = *(const u32x4p *)(B + row * ldb + 32 * t + 16 * c);
    *(u32x4p *)(Bp + 16 * o) = v;
}

hipError_t launch_prepack_b32(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp,
                              hipStream_t s)
{
    const int64_t nst = row_bytes / 32;
    const int64_t slots = (N + 31) / 32 * nst * 64;
    const int64_t grid = (slots + 255) / 256;
    if (grid >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prepack_b32_kernel, dim3((unsigned)grid), dim3(256), 0, s, B, ldb, N, nst, Bp, slots);
    return hipGetLastError();
}

hipError_t launch_prepack_b(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp,
                            hipStream_t s)
{
    const int64_t nst = row_bytes / 64;
    const int64_t slots = (N + 15) / 16 * nst * 64;
    const int64_t grid = (slots + 255) / 256;
    if (grid >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prepack_b_kernel, dim3((unsigned)grid), dim3(256), 0, s, B, ldb, N, nst, Bp, slots);
    return hipGetLastError();
}

}  // namespace qgemm
