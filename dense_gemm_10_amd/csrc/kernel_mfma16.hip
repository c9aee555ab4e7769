// Tile configurations and dispatch of the 16-bit matrix-core GEMM; the
// kernels are in mfma16.hpp, instantiated by the kernel_mfma16_*.hip files.
#include "mfma16.hpp"

namespace dg {

// variant index -> instantiation (BM x BN tile, WM x WN wavefronts, ring
// depth); the last field is mfma16_per_cu of the instantiation.
// Entries 0 and 1 are the large and small tiles of the automatic choice:
// 256 x 256 with whole-line (BK = 64) stages in a 2-stage ring and 16 x 16
// MFMA blocks, and 128 x 128 with BK = 32 in a 4-stage ring (64 KB of LDS,
// two workgroups per CU).  The others are selectable by name for sweeps.  The fp16 table
// has the same tiles.
#define DG_TILE16(T, BM, BN, BK, NS, V) \
    {BM, BN, BK, 256, V, "mfma_" #T "_" #BM "x" #BN "x" #BK "_w2x2_s" #NS, mfma16_per_cu(BM, BN, NS, BK)}
const TileConfig kMfmaBf16Tiles[] = {
    DG_TILE16(bf16, 256, 256, 64, 2, 5),
    DG_TILE16(bf16, 128, 128, 32, 4, 1),
    DG_TILE16(bf16, 256, 256, 32, 4, 0),
    DG_TILE16(bf16, 256, 128, 32, 4, 2),
    DG_TILE16(bf16, 256, 128, 32, 3, 3),
    DG_TILE16(bf16, 128, 256, 32, 3, 4),
    DG_TILE16(bf16, 128, 128, 64, 3, 6),
    DG_TILE16(bf16, 256, 128, 64, 3, 7),
    DG_TILE16(bf16, 128, 256, 32, 2, 8),
    DG_TILE16(bf16, 128, 128, 32, 2, 9),
};
const int kNumMfmaBf16Tiles = 10;

const TileConfig kMfmaF16Tiles[] = {
    DG_TILE16(f16, 256, 256, 64, 2, 5),
    DG_TILE16(f16, 128, 128, 32, 4, 1),
    DG_TILE16(f16, 256, 256, 32, 4, 0),
    DG_TILE16(f16, 256, 128, 32, 4, 2),
    DG_TILE16(f16, 256, 128, 32, 3, 3),
    DG_TILE16(f16, 128, 256, 32, 3, 4),
    DG_TILE16(f16, 128, 128, 64, 3, 6),
    DG_TILE16(f16, 256, 128, 64, 3, 7),
    DG_TILE16(f16, 128, 256, 32, 2, 8),
    DG_TILE16(f16, 128, 128, 32, 2, 9),
};
#undef DG_TILE16
const int kNumMfmaF16Tiles = 10;

hipError_t launch_mfma16(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const bool k_contiguous = g.a_col == 0 && g.b_col != 0;
    if (!k_contiguous) {
        // the planner keeps these layouts on the two tiles that have them
        if (p.tile.variant == 5)
            return launch_mfma16_mn256(g, p, stream);
        if (p.tile.variant == 1)
            return launch_mfma16_mn128(g, p, stream);
        return hipErrorInvalidValue;
    }
    if (g.ab_type == DT_F16)
        return p.tile.variant <= 4 ? launch_mfma16_f16_a(g, p, stream)
                                   : launch_mfma16_f16_b(g, p, stream);
    return p.tile.variant <= 4 ? launch_mfma16_bf16_a(g, p, stream)
                               : launch_mfma16_bf16_b(g, p, stream);
}

} // namespace dg
