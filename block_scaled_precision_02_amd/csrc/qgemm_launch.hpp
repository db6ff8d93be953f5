// qgemm_launch.hpp -- host-side launch of one kernel variant.
#pragma once
#include <hip/hip_runtime.h>
#include "qgemm_dma.hpp"
#include "qgemm_skinny.hpp"

namespace qgemm {

// Tile ids of the host table:
//   0 -> 256x256, 2x2 waves of 128x128 (1 wave per SIMD, 256 accumulators)
//   1 -> 128x128, 2x2 waves of 64x64
//   2 -> 256x256, 2x4 waves of 128x64 (2 waves per SIMD, 128 accumulators)
//   3 -> 192x192, 2x2 waves of 96x96 (144 accumulators)
//   4 -> 256x256 as tile 0, operands fetched straight into LDS (qgemm_dma.hpp);
//        needs K bytes % 64 == 0 and, for the scaled paths, K % 128 == 0 (the
//        e4m3-staged MX paths: K % 32, the SU form at K % 128 != 0)
//        with aligned scales
//   5 -> 256x256 fetched straight into LDS as tile 4, 2x4 waves of 128x64 (two
//        waves per SIMD); same requirements
//   6 -> 192x192 fetched straight into LDS, 2x2 waves of 96x96; same requirements
//   7 -> 128x128 fetched straight into LDS, 2x2 waves of 64x64; same requirements
//   8 -> small M (qgemm_skinny.hpp): 16 rows x 16 columns, eight waves splitting
//        K; bf16 output
//   9 -> small M: 64 rows x 16 columns, eight waves splitting K; same paths
//  10 -> FP8 blockscale only: 256 rows x 128 columns fetched straight into LDS,
//        2x2 waves of 128x64 (one wave per SIMD: 128 totals + 128 partial sums)
constexpr int NUM_TILES = 11;
constexpr int DMA_TILE = 4, DMA8_TILE = 5, DMA192_TILE = 6, DMA128_TILE = 7;
constexpr int SKINNY16_TILE = 8, SKINNY64_TILE = 9, F8B256_TILE = 10;
__host__ __device__ constexpr bool is_dma_tile(int tile) { return tile >= DMA_TILE && tile <= DMA128_TILE; }
__host__ __device__ constexpr bool is_skinny_tile(int tile) { return tile == SKINNY16_TILE || tile == SKINNY64_TILE; }
// Output rows (of A) and columns (rows of B) of one workgroup's tile.
__host__ __device__ constexpr int tile_edge_m(int tile)
{
    return tile == SKINNY16_TILE ? 16 : tile == SKINNY64_TILE ? 64
         : (tile == 1 || tile == DMA128_TILE) ? 128 : ((tile == 3 || tile == DMA192_TILE) ? 192 : 256);
}
__host__ __device__ constexpr int tile_edge_n(int tile)
{
    return is_skinny_tile(tile) ? 16 : tile == F8B256_TILE ? 128 : tile_edge_m(tile);
}
__host__ __device__ constexpr int tile_edge(int tile) { return tile_edge_m(tile); }
__host__ __device__ constexpr int tile_threads(int tile)
{
    return (tile == 2 || tile == DMA8_TILE || is_skinny_tile(tile)) ? 512 : 256;
}

template <int PATH, int WM, int WN, int TM, int TN, bool BIAS, int BROWS, bool SVEC, int OUT>
hipError_t launch_variant(const Params &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(64 * WM * WN);
    hipLaunchKernelGGL((qgemm_kernel<PATH, WM, WN, TM, TN, BIAS, BROWS, SVEC, OUT>), grid, block, 0, s, p);
    return hipGetLastError();
}

// The e4m3-staged MX paths at K % 128 != 0 (scale rows of K/32 bytes off
// dword boundaries; at K % 64 == 32 a last half stage): tiles 4, 5, 7, and 6
// for e4m3.
template <int PATH, bool BIAS, int BROWS, int OUT = OUT_BF16>
hipError_t launch_dma_su(int tile, const Params &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
    switch (tile) {
    case DMA_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 4, 4, BIAS, BROWS, OUT, true>), grid, block, 0, s, p);
        break;
    case DMA8_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 4, 4, 2, BIAS, BROWS, OUT, true>), grid, block, 0, s, p);
        break;
    case DMA192_TILE:
        if constexpr (PATH == PATH_MX8) {
            hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 3, 3, BIAS, BROWS, OUT, true>), grid, block, 0, s, p);
            break;
        } else {
            return hipErrorInvalidValue;
        }
    case DMA128_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 2, 2, BIAS, BROWS, OUT, true>), grid, block, 0, s, p);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int PATH, bool BIAS, int BROWS, bool SVEC, int OUT>
hipError_t launch_tile(int tile, const Params &p, hipStream_t s)
{
    switch (tile) {
    case 0: return launch_variant<PATH, 2, 2, 4, 4, BIAS, BROWS, SVEC, OUT>(p, s);
    case 1: return launch_variant<PATH, 2, 2, 2, 2, BIAS, BROWS, SVEC, OUT>(p, s);
    case 2: return launch_variant<PATH, 2, 4, 4, 2, BIAS, BROWS, SVEC, OUT>(p, s);
    case 3: return launch_variant<PATH, 2, 2, 3, 3, BIAS, BROWS, SVEC, OUT>(p, s);
    case DMA_TILE:
    case DMA8_TILE:
    case DMA192_TILE:
    case DMA128_TILE:
        if constexpr (PATH == PATH_MX8) {
            if (p.kblocks % 4 != 0)   // K % 128 != 0: scale rows off dword boundaries (any K/32)
                return launch_dma_su<PATH, BIAS, BROWS, OUT>(tile, p, s);
        }
        if constexpr (PATH == PATH_MX8 || PATH == PATH_MX4) {
            if (!SVEC)
                return hipErrorInvalidValue;
        }
        {
            const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
            if (tile == DMA_TILE)
                hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 4, 4, BIAS, BROWS, OUT>), grid, block, 0, s, p);
            else if (tile == DMA8_TILE)
                hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 4, 4, 2, BIAS, BROWS, OUT>), grid, block, 0, s, p);
            else if (tile == DMA192_TILE)
                hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 3, 3, BIAS, BROWS, OUT>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 2, 2, BIAS, BROWS, OUT>), grid, block, 0, s, p);
            return hipGetLastError();
        }
    case SKINNY16_TILE:
    case SKINNY64_TILE:
        if constexpr (OUT == OUT_BF16) {
            const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
            if (tile == SKINNY16_TILE)
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH, 1, skinny_depth<PATH, 1>(), BIAS, BROWS>), grid, block, 0,
                                   s, p);
            else
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH, 4, skinny_depth<PATH, 4>(), BIAS, BROWS>), grid, block, 0,
                                   s, p);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    default: return hipErrorInvalidValue;
    }
}

// Per-path entry points, one translation unit each.
hipError_t launch_i8(int tile, bool bias, int out, const Params &p, hipStream_t s);
hipError_t launch_f8(int tile, bool bias, const Params &p, hipStream_t s);
hipError_t launch_mx8(int tile, bool bias, int brows, bool svec, const Params &p, hipStream_t s);
hipError_t launch_mx4(int tile, bool bias, int brows, bool svec, const Params &p, hipStream_t s);
// FP8 blockscale: tiles 7 and 10, small-M tiles 8 and 9 (need K % 256 == 0 and
// 8-byte aligned scale arrays).
hipError_t launch_f8b(int tile, bool bias, const Params &p, hipStream_t s);
// MX with e4m3 A and e2m1 B: tiles 4, 5, 7 and small-M tiles 8, 9 (same
// requirements as MX on them).
hipError_t launch_mx84(int tile, bool bias, int brows, const Params &p, hipStream_t s);
// MX with e2m1 A and e4m3 B: tiles 4, 5, 7 (same requirements as MX on them).
hipError_t launch_mx48(int tile, bool bias, int brows, const Params &p, hipStream_t s);
// MX e2m1 at K % 128 != 0 in 64-element stages: tiles 4, 5, 7 (K/32 % 4 != 0).
hipError_t launch_mx4h(int tile, bool bias, int brows, const Params &p, hipStream_t s);
// MX with 6-bit elements (E2M3, or E3M2 when e3m2): tiles 4, 5, 7 (K % 128 == 0
// and 8-byte aligned scale arrays, as e4m3 MX on them).
hipError_t launch_mx6(int tile, bool e3m2, bool bias, int brows, const Params &p, hipStream_t s);

}  // namespace qgemm
