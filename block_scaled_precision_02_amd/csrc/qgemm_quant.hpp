// qgemm_quant.hpp -- launchers of the activation quantisers (qgemm_quant.hip).
// Arguments are checked by the C ABI before these are called: X 16-byte
// aligned with ldx a multiple of 8 elements, Q 16-byte aligned with ldq a
// multiple of 16 bytes, K a positive multiple of 32, M > 0.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qgemm {
// Per-token e4m3: Q [M,K] codes (row stride ldq bytes), scale [M] fp32.
hipError_t launch_quant_f8_pertoken(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *scale,
                                    int M, int K, hipStream_t s);
// Blockscale e4m3 (K % 128 == 0): Q [M,K] codes, S [M, K/128] fp32 with row
// stride lds elements.
hipError_t launch_quant_f8_block(const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, float *S, int64_t lds,
                                 int M, int K, hipStream_t s);
// MX, fmt 0 e4m3 (Q [M,K] bytes) or 1 e2m1 (Q [M,K/2] bytes); S [M,K/32]
// codes with row stride lds bytes.
hipError_t launch_quant_mx(int fmt, const uint16_t *X, int64_t ldx, uint8_t *Q, int64_t ldq, uint8_t *S,
                           int64_t lds, int M, int K, hipStream_t s);
}  // namespace qgemm
