// qgemm_pack.hpp -- launcher of the weight prepacking kernel (qgemm_pack.hip).
// Arguments are checked by the C ABI before it is called: B and Bp 16-byte
// aligned, ldb a multiple of 16 bytes and >= row_bytes, row_bytes a positive
// multiple of 256, N > 0.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qgemm {
hipError_t launch_prepack_b(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp,
                            hipStream_t s);
// The mixed MX GEMM's e2m1 B: 32-row groups of 32-byte pieces (row_bytes a
// positive multiple of 128).
hipError_t launch_prepack_b32(const uint8_t *B, int64_t ldb, int64_t N, int64_t row_bytes, uint8_t *Bp,
                              hipStream_t s);
}  // namespace qgemm
