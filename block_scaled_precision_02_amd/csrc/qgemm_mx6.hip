// MX variants with 6-bit elements (OCP FP6 E2M3 / E3M2), LDS-fetch kernel only:
// tiles 4 (256x256, four waves) and 7 (128x128).  Not built: the eight-wave
// 256x256 tile (its 256 registers a lane cannot hold the fragments' read
// offsets beside the accumulators: it spills) and 192x192 (a ring slot of 384
// rows x 64 bytes is not a power of two, which the FP6 ring addressing needs).
#include "qgemm_launch.hpp"

namespace qgemm {
template <int PATH, bool BIAS, int BROWS>
static hipError_t tiles(int tile, const Params &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(tile_threads(tile));
    switch (tile) {
    case DMA_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 4, 4, BIAS, BROWS, OUT_BF16>), grid, block, 0, s, p);
        break;
    case DMA128_TILE:
        hipLaunchKernelGGL((qgemm_dma_kernel<PATH, 2, 2, 2, BIAS, BROWS, OUT_BF16>), grid, block, 0, s, p);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int PATH>
static hipError_t by_bias(int tile, bool bias, int brows, const Params &p, hipStream_t s)
{
    if (brows == 1)
        return bias ? tiles<PATH, true, 1>(tile, p, s) : tiles<PATH, false, 1>(tile, p, s);
    return bias ? tiles<PATH, true, 32>(tile, p, s) : tiles<PATH, false, 32>(tile, p, s);
}

hipError_t launch_mx6(int tile, bool e3m2, bool bias, int brows, const Params &p, hipStream_t s)
{
    return e3m2 ? by_bias<PATH_MX6E3>(tile, bias, brows, p, s) : by_bias<PATH_MX6>(tile, bias, brows, p, s);
}
}  // namespace qgemm
