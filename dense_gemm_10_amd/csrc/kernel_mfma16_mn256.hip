// Instantiations of the 16-bit matrix-core GEMM (mfma16.hpp): an M- or N-contiguous operand, 256 x 256 tile
// on 16 x 16 x 32 MFMA blocks, bf16 and fp16.
#include "mfma16.hpp"

namespace dg {

template <int T>
hipError_t launch_mn256(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const bool at = g.a_col != 0, bt = g.b_col == 0;
    if (at && bt)
        return launch_layout<T, 256, 256, 2, 2, 2, 64, true, true, 16>(g, p, stream);
    if (at)
        return launch_layout<T, 256, 256, 2, 2, 2, 64, true, false, 16>(g, p, stream);
    return launch_layout<T, 256, 256, 2, 2, 2, 64, false, true, 16>(g, p, stream);
}

hipError_t launch_mfma16_mn256(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    return g.ab_type == DT_F16 ? launch_mn256<DT_F16>(g, p, stream)
                               : launch_mn256<DT_BF16>(g, p, stream);
}

} // namespace dg
