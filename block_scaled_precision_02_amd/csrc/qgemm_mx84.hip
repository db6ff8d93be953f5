// Mixed MX variants: e4m3 A (activations) with e2m1 B (weights), ue8m0 scales
// per 32 K elements on both (v_mfma_scale_f32_32x32x64_f8f6f4 with an FP4
// first operand and an FP8 second), run by the LDS-fetch kernel: tiles 4, 5
// and 7 (the 192x192 tile's B rows are not a whole number of 32-row fetches
// per wave); small M by the small-M kernel (tiles 8, 9).
#include "qgemm_launch.hpp"

namespace qgemm {
template <bool BIAS, int BROWS>
static hipError_t mx84_tile(int tile, const Params &p, hipStream_t s)
{
    if (is_dma_tile(tile) && p.kblocks % 4 != 0)   // K % 128 != 0
        return launch_dma_su<PATH_MX84, BIAS, BROWS>(tile, p, s);
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
    switch (tile) {
    case DMA_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_MX84, 2, 4, 4, BIAS, BROWS, OUT_BF16>), grid, block, 0, s, p);
        break;
    case DMA8_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_MX84, 4, 4, 2, BIAS, BROWS, OUT_BF16>), grid, block, 0, s, p);
        break;
    case DMA128_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH_MX84, 2, 2, 2, BIAS, BROWS, OUT_BF16>), grid, block, 0, s, p);
        break;
    case SKINNY16_TILE:
        hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_MX84, 1, skinny_depth<PATH_MX84, 1>(), BIAS, BROWS>), grid,
                           block, 0, s, p);
        break;
    case SKINNY64_TILE:
        hipLaunchKernelGGL((qgemm_skinny_kernel<PATH_MX84, 4, skinny_depth<PATH_MX84, 4>(), BIAS, BROWS>), grid,
                           block, 0, s, p);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mx84(int tile, bool bias, int brows, const Params &p, hipStream_t s)
{
    if (brows == 1)
        return bias ? mx84_tile<true, 1>(tile, p, s) : mx84_tile<false, 1>(tile, p, s);
    return bias ? mx84_tile<true, 32>(tile, p, s) : mx84_tile<false, 32>(tile, p, s);
}
}  // namespace qgemm
