// FP8 blockscale variants: e4m3 with fp32 scales per 128-element K block,
// applied inside the K loop of the LDS-fetch kernel (128x128 tile, four waves
// of 64x64: 64 partial-sum and 64 total registers per lane).
#include "qgemm_launch.hpp"

namespace qgemm {
hipError_t launch_f8b(int tile, bool bias, const Params &p, hipStream_t s)
{
    if (tile != DMA128_TILE)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
    if (bias)
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 2, 2, true, 128, OUT_BF16>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_F8B, 2, 2, 2, false, 128, OUT_BF16>), grid, block, 0, s, p);
    return hipGetLastError();
}
}  // namespace qgemm
