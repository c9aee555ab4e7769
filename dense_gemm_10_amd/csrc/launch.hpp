// Host-side plan and the launchers each kernel file provides.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dg {

enum Kernel {
    KERNEL_GENERIC = 1,
    KERNEL_VALU_F32 = 2,
    KERNEL_MFMA_BF16 = 3,
    KERNEL_MFMA_F32 = 4,
    KERNEL_MFMA_F16 = 5,
};

// One tile configuration of a kernel family.
struct TileConfig {
    int32_t bm, bn, bk;
    int32_t threads;
    int32_t variant;     // index into the family's instantiation table
    const char *name;
    int32_t per_cu;      // workgroups one CU holds at once (LDS and registers)
};

struct Plan {
    Kernel kernel;
    TileConfig tile;
    int32_t splits;          // >= 1
    int64_t k_per_split;
    int64_t programs;        // grid size of the main kernel
    size_t workspace_bytes;  // 0 unless splits > 1
    int64_t reduce_blocks;   // grid of the split-K reduction (0 if none)
    StreamK sk;              // sk.tail_tiles > 0: stream-K launch
    int64_t fixup_blocks;    // grid of the stream-K fix-up (0 if none)
    int32_t tuned;           // 1: tile and schedule from the offline-tuned table
};

// Whether the split-K reduction takes four outputs per thread (N a multiple
// of 4, every output index below 2^31); its grid is then a quarter as large.
inline bool reduce_by_four(int64_t N, int64_t total)
{
    return N % 4 == 0 && total < ((int64_t)1 << 31);
}

// Launchers: enqueue the kernel on `stream`; return hipSuccess or the
// launch error.
hipError_t launch_generic(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_valu_f32(const GemmArgs &g, const Plan &p, hipStream_t stream);
// bf16 and fp16 matrix-core kernels (element type from g.ab_type)
hipError_t launch_mfma16(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma_f32(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_splitk_reduce(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_streamk_fixup(const GemmArgs &g, const Plan &p, hipStream_t stream);
// Columns [n0, n0 + nrem) of the output (nrem <= kMaxSliver): a few rows
// of A per wavefront, row-major A with 16-byte aligned rows.
constexpr int kMaxSliver = 8;
constexpr int kSliverThreads = 256;        // 4 wavefronts per workgroup
constexpr int kSliverRows = 4;             // rows of A per wavefront
constexpr int kSliverRowsPerBlock = kSliverThreads / 64 * kSliverRows;
hipError_t launch_sliver(const GemmArgs &g, int64_t n0, int32_t nrem, hipStream_t stream);

// Tile configurations of each family (defined next to the kernels).
extern const TileConfig kGenericTiles[];
extern const TileConfig kValuTiles[];
extern const TileConfig kMfmaBf16Tiles[];
extern const TileConfig kMfmaF32Tiles[];
extern const TileConfig kMfmaF16Tiles[];
extern const int kNumGenericTiles, kNumValuTiles, kNumMfmaBf16Tiles, kNumMfmaF32Tiles,
    kNumMfmaF16Tiles;

} // namespace dg
