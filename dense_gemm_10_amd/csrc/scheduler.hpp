// Output-tile scheduler shared by every GEMM kernel and by the host-side
// map check (dg_schedule_map).  Compiled for host and device from the same
// source so the CPU test exercises exactly what the kernels run.
//
// A launch has P = batch * splits * T programs, T = num_pid_m * num_pid_n
// output tiles of BM x BN (ceil-div counts, so ragged tiles are included:
// "Skill: Write a Triton GEMM Kernel", Required reasoning process step 2
// and the grid-size failure mode).  Program id -> (b, s, pid_m, pid_n) is
// the composition of three bijections:
//   1. XCD remap.  The hardware deals consecutive workgroup ids round-robin
//      to the 8 XCDs of an MI355X, each with its own L2.  Program p runs on
//      XCD x = p mod 8; it is given logical id x*q + min(x, r) + p/8 with
//      q = P/8, r = P mod 8, so XCD x owns one contiguous run of logical ids
//      and the grouped order below stays local to one L2.
//   2. Decode of the logical id L: t = L mod T, then split s, then batch b
//      (tiles of one (b, s) are consecutive).
//   3. Grouped tile order ("GEMM Kernel Optimization", L2 Cache Grouping;
//      "Skill: Write a Triton GEMM Kernel", Required reasoning process
//      step 2): the tile rows are cut into bands of G rows (the last band
//      may be shorter), the bands are taken top to bottom, and inside a
//      band the tiles are taken column by column, top to bottom within a
//      column.  A run of consecutive programs then reuses the same few A
//      row panels and B column panels instead of sweeping a whole tile row.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define DG_HD __host__ __device__
#else
#define DG_HD
#endif

namespace dg {

constexpr int kNumXcd = 8;

struct SchedArgs {
    int64_t num_pid_m, num_pid_n;  // output tiles along M and N
    int64_t batch;
    int32_t splits;                // split-K slices (>= 1)
    int32_t group_m;               // >= 1
    int32_t xcd_remap;             // 1 = on
    int32_t pad_;
};

struct TileCoord {
    int64_t b;
    int32_t s;
    int32_t pid_m;
    int32_t pid_n;
};

DG_HD inline int64_t sched_programs(const SchedArgs &a)
{
    return a.batch * (int64_t)a.splits * a.num_pid_m * a.num_pid_n;
}

DG_HD inline int64_t xcd_remap(int64_t pid, int64_t P)
{
    int64_t x = pid % kNumXcd;
    int64_t q = P / kNumXcd, r = P % kNumXcd;
    return x * q + (x < r ? x : r) + pid / kNumXcd;
}

// Grouped order of tile index t (0 <= t < num_pid_m * num_pid_n) ->
// (pid_m, pid_n); b and s are left 0.  Band `band` holds tile rows
// [band * G, band * G + h) with h = min(G, rows left) and its h * num_pid_n
// tiles; position o inside the band walks column o / h, row o mod h.
DG_HD inline TileCoord decode_tile(int64_t t, const SchedArgs &a)
{
    const int64_t G = a.group_m;
    const int64_t band_tiles = G * a.num_pid_n;      // tiles of a full band
    const int64_t band = t / band_tiles;
    const int64_t o = t - band * band_tiles;         // position inside the band
    const int64_t row0 = band * G;
    const int64_t left = a.num_pid_m - row0;
    const int64_t h = left < G ? left : G;           // rows in this band
    TileCoord c;
    c.b = 0;
    c.s = 0;
    c.pid_m = (int32_t)(row0 + o % h);
    c.pid_n = (int32_t)(o / h);
    return c;
}

DG_HD inline TileCoord decode_program(int64_t pid, const SchedArgs &a)
{
    const int64_t T = a.num_pid_m * a.num_pid_n;
    const int64_t P = a.batch * (int64_t)a.splits * T;
    const int64_t L = a.xcd_remap ? xcd_remap(pid, P) : pid;
    const int64_t bs = L / T;
    TileCoord c = decode_tile(L % T, a);
    c.s = (int32_t)(bs % a.splits);
    c.b = bs / a.splits;
    return c;
}

// Stream-K tail (one matrix, no split-K): the tiles of the full waves,
// [0, dp_tiles), are computed whole by programs [0, dp_tiles); each of the
// tail_tiles remaining tiles has its K range cut into tail_splits slices of
// k_per_split (a multiple of the kernel's BK), one program per slice, which
// writes a raw fp32 partial.  Tail program i (0 <= i < tail_tiles *
// tail_splits, after the XCD remap) takes slice i / tail_tiles of tail tile
// i % tail_tiles: programs with the same slice read the same K range of
// their A and B panels.
struct StreamK {
    int64_t dp_tiles;
    int64_t tail_tiles;       // 0: plain data-parallel launch
    int64_t tail_splits;
    int64_t k_per_split;
};

} // namespace dg
