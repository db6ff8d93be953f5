// FP8 e4m3 per-token / per-channel variants (unscaled v_mfma_f32_32x32x64_f8f6f4).
#include "qgemm_launch.hpp"

namespace qgemm {
hipError_t launch_f8(int tile, bool bias, const Params &p, hipStream_t s)
{
    return bias ? launch_tile<PATH_F8, true, 1, false, OUT_BF16>(tile, p, s)
                : launch_tile<PATH_F8, false, 1, false, OUT_BF16>(tile, p, s);
}
}  // namespace qgemm
