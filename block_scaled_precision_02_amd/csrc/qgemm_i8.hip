// INT8 rowwise variants (v_mfma_i32_32x32x32_i8, int32 accumulators).
#include "qgemm_launch.hpp"

namespace qgemm {
hipError_t launch_i8(int tile, bool bias, int out, const Params &p, hipStream_t s)
{
    if (out == OUT_I32)
        return launch_tile<PATH_I8, false, 1, false, OUT_I32>(tile, p, s);
    return bias ? launch_tile<PATH_I8, true, 1, false, OUT_BF16>(tile, p, s)
                : launch_tile<PATH_I8, false, 1, false, OUT_BF16>(tile, p, s);
}
}  // namespace qgemm
