// MX variants, e2m1 elements (v_mfma_scale_f32_32x32x64_f8f6f4).
#include "qgemm_launch.hpp"

namespace qgemm {
template <bool BIAS, int BROWS>
static hipError_t by_svec(int tile, bool svec, const Params &p, hipStream_t s)
{
    return svec ? launch_tile<PATH_MX4, BIAS, BROWS, true, OUT_BF16>(tile, p, s)
                : launch_tile<PATH_MX4, BIAS, BROWS, false, OUT_BF16>(tile, p, s);
}

hipError_t launch_mx4(int tile, bool bias, int brows, bool svec, const Params &p, hipStream_t s)
{
    if (brows == 1)
        return bias ? by_svec<true, 1>(tile, svec, p, s) : by_svec<false, 1>(tile, svec, p, s);
    return bias ? by_svec<true, 32>(tile, svec, p, s) : by_svec<false, 32>(tile, svec, p, s);
}
}  // namespace qgemm
