// Instantiations of the 16-bit matrix-core GEMM (mfma16.hpp): bf16, K-contiguous operands, tile variants 5 to 9
// (variant 5, the 256 x 256 tile, on 16 x 16 x 32 MFMA blocks).
#include "mfma16.hpp"

namespace dg {

hipError_t launch_mfma16_bf16_b(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 5: return launch_one<DT_BF16, 256, 256, 2, 2, 2, 64, 16>(g, p, stream);
    case 6: return launch_one<DT_BF16, 128, 128, 2, 2, 3, 64>(g, p, stream);
    case 7: return launch_one<DT_BF16, 256, 128, 2, 2, 3, 64>(g, p, stream);
    case 8: return launch_one<DT_BF16, 128, 256, 2, 2, 2, 32>(g, p, stream);
    case 9: return launch_one<DT_BF16, 128, 128, 2, 2, 2, 32>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
