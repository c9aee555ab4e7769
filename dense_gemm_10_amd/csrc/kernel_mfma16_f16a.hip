// Instantiations of the 16-bit matrix-core GEMM (mfma16.hpp): fp16, K-contiguous operands, tile variants 0 to 4.
#include "mfma16.hpp"

namespace dg {

hipError_t launch_mfma16_f16_a(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 0: return launch_one<DT_F16, 256, 256, 2, 2, 4, 32>(g, p, stream);
    case 1: return launch_one<DT_F16, 128, 128, 2, 2, 4, 32>(g, p, stream);
    case 2: return launch_one<DT_F16, 256, 128, 2, 2, 4, 32>(g, p, stream);
    case 3: return launch_one<DT_F16, 256, 128, 2, 2, 3, 32>(g, p, stream);
    case 4: return launch_one<DT_F16, 128, 256, 2, 2, 3, 32>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
