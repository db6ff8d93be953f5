// MX e2m1 at K % 128 != 0: both operands staged 64 K elements (32 bytes a
// row) at a time, as the mixed paths stage their e2m1 operand (the e2m1
// kernel's 64-byte stages would leave part of one); scale rows of K/32 bytes
// off dword boundaries, and at K % 64 == 32 a last half stage, take the SU
// form.
// Tiles 4, 5 and 7 (the 192x192 tile's rows are not a whole number of
// 32-row fetches per wave).
#include "qgemm_launch.hpp"

namespace qgemm {
hipError_t launch_mx4h(int tile, bool bias, int brows, const Params &p, hipStream_t s)
{
    if (tile != DMA_TILE && tile != DMA8_TILE && tile != DMA128_TILE)
        return hipErrorInvalidValue;
    if (brows == 1)
        return bias ? launch_dma_su<PATH_MX4H, true, 1>(tile, p, s) : launch_dma_su<PATH_MX4H, false, 1>(tile, p, s);
    return bias ? launch_dma_su<PATH_MX4H, true, 32>(tile, p, s) : launch_dma_su<PATH_MX4H, false, 32>(tile, p, s);
}
}  // namespace qgemm
