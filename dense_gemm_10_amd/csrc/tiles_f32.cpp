// Tile configurations of the fp32 matrix-core kernel (kernel_mfma_f32.hip),
// kept apart from the kernels so that host code can be built without them.
// Variant v is the instantiation launch_mfma_f32 runs for it.
#include "launch.hpp"

namespace dg {

const TileConfig kMfmaF32Tiles[] = {
    {256, 256, 16, 256, 0, "mfma_f32_256x256x16_w2x2"},
    {128, 128, 16, 256, 1, "mfma_f32_128x128x16_w2x2"},
    {256, 256, 32, 256, 2, "mfma_f32_256x256x32_w2x2"},
    {128, 128, 32, 256, 3, "mfma_f32_128x128x32_w2x2"},
};
const int kNumMfmaF32Tiles = 4;

} // namespace dg
