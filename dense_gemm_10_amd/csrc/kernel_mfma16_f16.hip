// Instantiations of the 16-bit matrix-core GEMM (mfma16.hpp): fp16, K-contiguous operands.
#include "mfma16.hpp"

namespace dg {

hipError_t launch_mfma16_f16(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 1: return launch_one<DT_F16, 128, 128, 2, 2, 4, 32>(g, p, stream);
    case 5: return launch_one<DT_F16, 256, 256, 2, 2, 2, 64>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
