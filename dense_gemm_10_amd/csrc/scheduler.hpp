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
//
// A launch has at most 2^31 - 1 programs, so the decode runs in 32-bit
// unsigned arithmetic, and its divisions by the launch's counts (tiles per
// matrix, tiles per band, band height, splits) are a multiply-high and two
// shifts by constants the host prepares (sched_prepare): all scalar
// instructions, where a division by a value known only at run time is a
// chain of vector-to-scalar steps that delays a workgroup's first loads.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define DG_HD __host__ __device__
#else
#define DG_HD
#endif

namespace dg {

constexpr int kNumXcd = 8;

// Division of any 32-bit n by an invariant d >= 1: with l = ceil(log2 d)
// and m = floor(2^32 (2^l - d) / d) + 1 (which fits in 32 bits),
// n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), t = mulhi(m, n)
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, section 4, the unsigned case).
// sh holds min(l, 1) in bit 8 and max(l - 1, 0) below it; d itself is
// kept by the caller.
struct FastDiv {
    uint32_t m, sh;
};

DG_HD inline uint32_t fastdiv(uint32_t n, const FastDiv &f)
{
    const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
    return (t + ((n - t) >> (f.sh >> 8))) >> (f.sh & 0xff);
}

struct SchedArgs {
    int64_t num_pid_m, num_pid_n;  // output tiles along M and N
    int64_t batch;
    int32_t splits;                // split-K slices (>= 1)
    int32_t group_m;               // >= 1
    int32_t xcd_remap;             // 1 = on
    int32_t pad_;
    // filled by sched_prepare from the fields above: division by
    FastDiv by_tiles;              // num_pid_m * num_pid_n
    FastDiv by_band;               // group_m * num_pid_n, the tiles of a full band
    FastDiv by_group;              // group_m, the rows of a full band
    FastDiv by_last;               // the rows of the last band
    FastDiv by_splits;             // splits
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

inline FastDiv fastdiv_make(uint32_t d)
{
    if (d == 0)
        d = 1;     // a count of zero means an empty launch, which decodes nothing
    uint32_t l = 0;
    while (l < 32 && (1ull << l) < d)
        ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, (l < 1 ? l : 1u) << 8 | (l > 1 ? l - 1 : 0u)};
}

// The divisors of a launch whose program count fits in 31 bits.
inline void sched_prepare(SchedArgs &a)
{
    const int64_t G = a.group_m;
    const int64_t bands = (a.num_pid_m + G - 1) / G;
    a.by_tiles = fastdiv_make((uint32_t)(a.num_pid_m * a.num_pid_n));
    a.by_band = fastdiv_make((uint32_t)(G * a.num_pid_n));
    a.by_group = fastdiv_make((uint32_t)G);
    a.by_last = fastdiv_make((uint32_t)(bands > 0 ? a.num_pid_m - (bands - 1) * G : 1));
    a.by_splits = fastdiv_make((uint32_t)a.splits);
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
DG_HD inline TileCoord decode_tile(int64_t t64, const SchedArgs &a)
{
    const uint32_t t = (uint32_t)t64;
    const uint32_t G = (uint32_t)a.group_m;
    const uint32_t band = fastdiv(t, a.by_band);
    const uint32_t o = t - band * (G * (uint32_t)a.num_pid_n);   // position inside the band
    const uint32_t row0 = band * G;
    // rows in this band: G, or what is left for the last band
    const uint32_t left = (uint32_t)a.num_pid_m - row0;
    const bool last = left < G;
    const uint32_t h = last ? left : G;
    const FastDiv fh{last ? a.by_last.m : a.by_group.m, last ? a.by_last.sh : a.by_group.sh};
    const uint32_t col = fastdiv(o, fh);
    TileCoord c;
    c.b = 0;
    c.s = 0;
    c.pid_m = (int32_t)(row0 + (o - col * h));
    c.pid_n = (int32_t)col;
    return c;
}

DG_HD inline TileCoord decode_program(int64_t pid64, const SchedArgs &a)
{
    const uint32_t pid = (uint32_t)pid64;
    const uint32_t T = (uint32_t)a.num_pid_m * (uint32_t)a.num_pid_n;
    const uint32_t P = (uint32_t)a.batch * (uint32_t)a.splits * T;
    uint32_t L = pid;
    if (a.xcd_remap) {
        const uint32_t x = pid % kNumXcd, q = P / kNumXcd, r = P % kNumXcd;
        L = x * q + (x < r ? x : r) + pid / kNumXcd;
    }
    const uint32_t bs = fastdiv(L, a.by_tiles);
    TileCoord c = decode_tile(L - bs * T, a);
    const uint32_t b = fastdiv(bs, a.by_splits);
    c.s = (int32_t)(bs - b * (uint32_t)a.splits);
    c.b = b;
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
