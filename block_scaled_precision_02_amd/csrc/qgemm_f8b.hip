// FP8 blockscale variants: e4m3 with fp32 scales per 128-element K block,
// applied inside the K loop of the LDS-fetch kernel: tile 7 (128x128, four
// waves of 64x64: 64 partial-sum and 64 total registers per lane, two
// workgroups per CU) or tile 10 (256x128, four waves of 128x64: 128 + 128,
// one workgroup per CU); small M: the small-M kernel (tiles 8, 9).
#include "qgemm_launch.hpp"

namespace qgemm {
hipError_t launch_f8b(int tile, bool bias, const Params &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
    if (tile == SKINNY16_TILE || tile == SKINNY64_TILE) {
        constexpr int D1 = skinny_depth<PATH_F8B, 1>(), D4 = skinny_depth<PATH_F8B, 4>();
        if (tile == SKINNY16_TILE) {
            if (bias)
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_F8B, 1, D1, true, 128>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_F8B, 1, D1, false, 128>), grid, block, 0, s, p);
        } else {
            if (bias)
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_F8B, 4, D4, true, 128>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_F8B, 4, D4, false, 128>), grid, block, 0, s, p);
        }
        return hipGetLastError();
    }
    if (tile == F8B256_TILE) {
        if (bias)
            hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 4, 2, true, 128, OUT_BF16>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 4, 2, false, 128, OUT_BF16>), grid, block, 0, s, p);
        return hipGetLastError();
    }
    if (tile != DMA128_TILE)
        return hipErrorInvalidValue;
    if (bias)
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 2, 2, true, 128, OUT_BF16>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 2, 2, false, 128, OUT_BF16>), grid, block, 0, s, p);
    return hipGetLastError();
}
}  // namespace qgemm
