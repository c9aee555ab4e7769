// C ABI of the GEMM library: host-side validation (no HIP calls), plan
// selection (kernel family, tile, split-K, grid) and launches.
//
// Launcher behaviour follows "Skill: Write a Triton GEMM Kernel" (Output
// format: compute the grid, deal with strides; Common failure modes: the
// grid uses ceiling division, strides are never recomputed from shapes),
// the problem statement of "La GEMM, de zero a cuBLAS" section 2.1, and the
// split-K rule of the Skill page's kernel design rules (split K only when
// the output tiles alone cannot fill the GPU and K is long; partials go
// to a workspace and a separate pass reduces them).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/densegemm.h"
#include "launch.hpp"

using namespace dg;

static_assert(DT_F32 == DG_F32 && DT_BF16 == DG_BF16 && DT_F16 == DG_F16,
              "kernel dtype codes follow dg_dtype");

namespace {

constexpr int64_t kNumCu = 256;          // MI355X compute units
// Group height of the grouped tile order ("GEMM Kernel Optimization", L2
// Cache Grouping, which starts from 8).  4 with the XCD remap gives each
// XCD's 32 concurrent 256 x 256 tiles a 4 x 8 block of the tile grid: the
// fewest A and B panels, so the fewest L2 misses, of the group heights 1,
// 4, 8 and 16 with and without the remap.  The tile-order ablation
// (bench.py --ablation) measures the misses and the time of each order at
// 4096^3 and 8192^3.
constexpr int32_t kDefaultGroupM = 4;
constexpr int32_t kMaxSplits = 256;

int64_t elem_size(int32_t t) { return t == DG_F32 ? 4 : 2; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_add_overflow(a, b, out); }

// Elements spanned by one rows x cols matrix with the given order and ld.
bool matrix_span(int32_t order, int64_t rows, int64_t cols, int64_t ld, int64_t *span)
{
    if (rows == 0 || cols == 0) {
        *span = 0;
        return true;
    }
    int64_t outer = order == DG_ROW_MAJOR ? rows : cols;
    int64_t inner = order == DG_ROW_MAJOR ? cols : rows;
    int64_t t;
    return mul_ok(outer - 1, ld, &t) && add_ok(t, inner, span);
}

// Elements spanned by the whole batch.
bool batch_span(int64_t span, int64_t batch, int64_t stride, int64_t *total)
{
    if (span == 0 || batch == 0) {
        *total = 0;
        return true;
    }
    int64_t t;
    return mul_ok(batch - 1, stride, &t) && add_ok(t, span, total);
}

struct Extents {
    int64_t a_bytes, b_bytes, c_bytes, bias_bytes;
    int64_t c_span;
};

bool ranges_overlap(const void *p, int64_t pn, const void *q, int64_t qn)
{
    if (!p || !q || pn <= 0 || qn <= 0)
        return false;
    uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pn;
    uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qn;
    return a0 < b1 && b0 < a1;
}

bool is_noop(const dg_gemm_desc *d) { return d->M == 0 || d->N == 0 || d->batch == 0; }

bool reads_ab(const dg_gemm_desc *d) { return d->alpha != 0.0f && d->K > 0; }

// Descriptor checks.  No HIP call is made here.
dg_status validate_desc(const dg_gemm_desc *d, Extents *ext)
{
    if (!d || d->struct_size != sizeof(dg_gemm_desc))
        return DG_ERROR_INVALID_VALUE;
    if (d->M < 0 || d->N < 0 || d->K < 0 || d->batch < 0)
        return DG_ERROR_INVALID_VALUE;
    auto dtype_ok = [](int32_t t) { return t == DG_F32 || t == DG_BF16 || t == DG_F16; };
    auto order_ok = [](int32_t o) { return o == DG_ROW_MAJOR || o == DG_COL_MAJOR; };
    if (!dtype_ok(d->a_type) || !dtype_ok(d->b_type) || !dtype_ok(d->c_type))
        return DG_ERROR_INVALID_VALUE;
    if (!order_ok(d->a_order) || !order_ok(d->b_order) || !order_ok(d->c_order))
        return DG_ERROR_INVALID_VALUE;
    if (d->act < DG_ACT_NONE || d->act > DG_ACT_GELU_TANH)
        return DG_ERROR_INVALID_VALUE;
    if (d->algo < DG_ALGO_AUTO || d->algo > DG_ALGO_MFMA_F16)
        return DG_ERROR_INVALID_VALUE;
    if (d->split_k < 0 || d->group_m < 0 || d->xcd_remap < -1 || d->xcd_remap > 1)
        return DG_ERROR_INVALID_VALUE;
    if (d->schedule < DG_SCHED_AUTO || d->schedule > DG_SCHED_STREAM_K)
        return DG_ERROR_INVALID_VALUE;
    if (d->bias && !dtype_ok(d->bias_type))
        return DG_ERROR_INVALID_VALUE;
    if (d->lda < 1 || d->ldb < 1 || d->ldc < 1)
        return DG_ERROR_INVALID_VALUE;
    if (d->stride_a < 0 || d->stride_b < 0 || d->stride_c < 0)
        return DG_ERROR_INVALID_VALUE;
    // leading dimension >= length of the contiguous dimension
    if (d->lda < (d->a_order == DG_ROW_MAJOR ? d->K : d->M))
        return DG_ERROR_INVALID_VALUE;
    if (d->ldb < (d->b_order == DG_ROW_MAJOR ? d->N : d->K))
        return DG_ERROR_INVALID_VALUE;
    if (d->ldc < (d->c_order == DG_ROW_MAJOR ? d->N : d->M))
        return DG_ERROR_INVALID_VALUE;
    // supported dtype combinations: A and B of one type; fp32 inputs give
    // an fp32 output, 16-bit inputs any output type
    if (d->a_type != d->b_type)
        return DG_ERROR_NOT_SUPPORTED;
    if (d->a_type == DG_F32 && d->c_type != DG_F32)
        return DG_ERROR_NOT_SUPPORTED;
    if (d->split_k > kMaxSplits)
        return DG_ERROR_NOT_SUPPORTED;

    int64_t sa, sb, sc, ta, tb, tc;
    if (!matrix_span(d->a_order, d->M, d->K, d->lda, &sa) ||
        !matrix_span(d->b_order, d->K, d->N, d->ldb, &sb) ||
        !matrix_span(d->c_order, d->M, d->N, d->ldc, &sc))
        return DG_ERROR_INVALID_VALUE;
    if (!batch_span(sa, d->batch, d->stride_a, &ta) || !batch_span(sb, d->batch, d->stride_b, &tb) ||
        !batch_span(sc, d->batch, d->stride_c, &tc))
        return DG_ERROR_INVALID_VALUE;
    // C matrices of different batch entries must not overlap
    if (d->batch > 1 && sc > 0 && d->stride_c < sc)
        return DG_ERROR_INVALID_VALUE;
    int64_t ab, bb, cb;
    if (!mul_ok(ta, elem_size(d->a_type), &ab) || !mul_ok(tb, elem_size(d->b_type), &bb) ||
        !mul_ok(tc, elem_size(d->c_type), &cb))
        return DG_ERROR_INVALID_VALUE;
    // work size must be addressable
    int64_t mn, bmn;
    if (!mul_ok(d->M, d->N, &mn) || !mul_ok(mn, d->batch, &bmn))
        return DG_ERROR_INVALID_VALUE;
    if (ext) {
        ext->a_bytes = ab;
        ext->b_bytes = bb;
        ext->c_bytes = cb;
        ext->bias_bytes = d->bias ? d->N * elem_size(d->bias_type) : 0;
        ext->c_span = sc;
    }
    return DG_SUCCESS;
}

dg_status validate_ptrs(const dg_gemm_desc *d, const Extents &e, const void *A, const void *B,
                        const void *C)
{
    if (is_noop(d))
        return DG_SUCCESS;
    if (!C)
        return DG_ERROR_INVALID_VALUE;
    if (reads_ab(d) && (!A || !B))
        return DG_ERROR_INVALID_VALUE;
    auto aligned = [](const void *p, int64_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; };
    if (!aligned(A, elem_size(d->a_type)) || !aligned(B, elem_size(d->b_type)) ||
        !aligned(C, elem_size(d->c_type)) || (d->bias && !aligned(d->bias, elem_size(d->bias_type))))
        return DG_ERROR_INVALID_VALUE;
    if (reads_ab(d) &&
        (ranges_overlap(C, e.c_bytes, A, e.a_bytes) || ranges_overlap(C, e.c_bytes, B, e.b_bytes)))
        return DG_ERROR_INVALID_VALUE;
    if (ranges_overlap(C, e.c_bytes, d->bias, e.bias_bytes))
        return DG_ERROR_INVALID_VALUE;
    return DG_SUCCESS;
}

bool aligned_to(const void *p, int64_t bytes) { return ((uintptr_t)p % bytes) == 0; }

// Batch strides keep every batch entry's A and B 16-byte aligned (they are
// not used when batch == 1).
bool strides_aligned(const dg_gemm_desc *d, int64_t elems)
{
    return d->batch <= 1 || (d->stride_a % elems == 0 && d->stride_b % elems == 0);
}

// Eligibility of the specialised kernels.  Pointers may be NULL (query
// without buffers): they then count as aligned.
bool valu_eligible(const dg_gemm_desc *d, const void *A, const void *B)
{
    if (d->a_type != DG_F32)
        return false;
    return aligned_to(A, 16) && aligned_to(B, 16) && d->lda % 4 == 0 && d->ldb % 4 == 0 &&
           strides_aligned(d, 4);
}

// bf16 or fp16 (`type`) matrix-core kernel, any order of A and B
bool mfma16_eligible(const dg_gemm_desc *d, int32_t type, const void *A, const void *B)
{
    if (d->a_type != type)
        return false;
    // the kernel addresses a tile with 32-bit byte offsets: 256 rows * ld * 2 < 2^31
    return aligned_to(A, 16) && aligned_to(B, 16) && d->lda % 8 == 0 && d->ldb % 8 == 0 &&
           strides_aligned(d, 8) && d->lda < (1 << 22) && d->ldb < (1 << 22);
}

// A row-major and B column-major: both operands K-contiguous, the layout
// every 16-bit tile configuration (and the tuned table) serves.  The other
// three run on the two tiles of the automatic choice.
bool k_contiguous(const dg_gemm_desc *d)
{
    return d->a_order == DG_ROW_MAJOR && d->b_order == DG_COL_MAJOR;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t tiles_of(const dg_gemm_desc *d, const TileConfig &t)
{
    return ceil_div(d->M, t.bm) * ceil_div(d->N, t.bn) * d->batch;
}

// Tile named by the DG_FORCE_TILE environment variable (benchmarking and
// ablation only), or NULL.
const TileConfig *forced_tile(const TileConfig *table, int n)
{
    const char *want = getenv("DG_FORCE_TILE");
    if (!want || !*want)
        return nullptr;
    for (int i = 0; i < n; ++i)
        if (strcmp(table[i].name, want) == 0)
            return &table[i];
    return nullptr;
}

// Offline-tuned plans, generated by dense_gemm_10_amd/tune.py from timed
// sweeps on an MI355X over every tile configuration of a family and both
// schedules ("GEMM Kernel Optimization", Autotune Configs, and "Skill:
// Write a Triton GEMM Kernel", Required reasoning process step 7: time the
// candidate configurations per problem size and keep the fastest; here the
// sweep runs once, offline, and its winners are compiled in, so no call
// ever benchmarks).  An exact (family, M, N, K, batch) match replaces the
// heuristic tile choice and states the schedule and the split-K count; the
// table ends with an entry whose tile is NULL.  DG_TUNED=0 in the environment switches it off
// (benchmarking and ablation only).
struct TunedEntry {
    int32_t kernel;
    int64_t M, N, K, batch;
    const char *tile;
    int32_t schedule;     // DG_SCHED_DATA_PARALLEL or DG_SCHED_STREAM_K
    int32_t splits;       // split-K slices (data-parallel) or K slices per tail
                          // tile (stream-K); 0: the automatic choice
};

const TunedEntry kTuned[] = {
#include "tuned_table.inc"
    {0, 0, 0, 0, 0, nullptr, 0, 0},
};

const TileConfig *tile_named(const TileConfig *table, int n, const char *name)
{
    for (int i = 0; i < n; ++i)
        if (strcmp(table[i].name, name) == 0)
            return &table[i];
    return nullptr;
}

// DG_FORCE_PLAN=<tile>:<dp|sk>:<splits> (the offline tuning sweep): an
// entry for any problem on the tile's family, applied exactly as a tuned
// entry is.  False when unset or when the tile is not in `table`.
bool forced_plan(const TileConfig *table, int n, Kernel k, TunedEntry *out)
{
    thread_local static char name[96];   // the entry points at it; one per planning thread
    const char *env = getenv("DG_FORCE_PLAN");
    if (!env)
        return false;
    const char *c1 = strchr(env, ':');
    const char *c2 = c1 ? strchr(c1 + 1, ':') : nullptr;
    if (!c1 || !c2 || c1 - env >= (ptrdiff_t)sizeof name)
        return false;
    memcpy(name, env, c1 - env);
    name[c1 - env] = 0;
    if (!tile_named(table, n, name))
        return false;
    memset(out, 0, sizeof *out);
    out->kernel = k;
    out->tile = name;
    out->schedule = strncmp(c1 + 1, "sk", 2) == 0 ? DG_SCHED_STREAM_K : DG_SCHED_DATA_PARALLEL;
    out->splits = atoi(c2 + 1);
    return true;
}

// The tuned entry for this problem on kernel family k whose tile exists in
// `table`, or NULL.
const TunedEntry *find_tuned(const dg_gemm_desc *d, Kernel k, const TileConfig *table, int n)
{
    const char *off = getenv("DG_TUNED");
    if (off && strcmp(off, "0") == 0)
        return nullptr;
    for (const TunedEntry *e = kTuned; e->tile; ++e)
        if (e->kernel == k && e->M == d->M && e->N == d->N && e->K == d->K &&
            e->batch == d->batch && tile_named(table, n, e->tile))
            return e;
    return nullptr;
}

// Pick the matrix-core tile.  The 256 x 256 tile (one workgroup per CU) has
// the best flop-per-byte ratio but quantises badly when its tile count is
// not close to a whole number of waves over the 256 CUs ("La GEMM, de zero
// a cuBLAS", section 2.10 on wave quantisation): e.g. 4095 x 4097 gives 272
// tiles = 1.06 waves.  It is used only when the waves it forms are at least
// 85 % full; otherwise the 128 x 128 tile (two workgroups per CU, 4x the
// tiles) is used.
TileConfig pick_quantised(const dg_gemm_desc *d, const TileConfig *table, int n)
{
    if (const TileConfig *f = forced_tile(table, n))
        return *f;
    const TileConfig &t256 = table[0], &t128 = table[1];
    // A flat GEMM (K of one or two K steps, "La GEMM, de zero a cuBLAS",
    // self-check on 4096 x 4096 x 16) is bound by writing C: more, smaller
    // tiles keep more stores in flight (measured 20 vs 25 us in bf16, 25.5
    // vs 30 us in fp32 at 4096 x 4096 x 16).
    if (d->K <= 64)
        return t128;
    const int64_t tiles = tiles_of(d, t256);
    const int64_t waves = ceil_div(tiles, kNumCu);
    if (tiles >= kNumCu && tiles * 100 >= waves * kNumCu * 85)
        return t256;
    return t128;
}


// Split-K slices for `tiles` output tiles: only when the tiles alone leave
// most compute units idle and every slice keeps a long K range: 1024 for
// 16-bit inputs, 256 for fp32, whose K steps cost 8 to 16 times more
// matrix-core time per element (measured at 1024^3 fp32: 42 us in 4 slices
// against 112 us unsplit).
int32_t auto_splits(const dg_gemm_desc *d, int64_t tiles)
{
    const int64_t min_slice = d->a_type == DG_F32 ? 256 : 1024;
    if (!reads_ab(d) || tiles >= kNumCu / 2 || d->K < 2 * min_slice)
        return 1;
    int64_t s = kNumCu / tiles;                  // about one program per CU
    int64_t by_k = d->K / min_slice;             // keep >= min_slice of K per slice
    if (s > by_k) s = by_k;
    if (s > 16) s = 16;
    return s < 2 ? 1 : (int32_t)s;
}

// Split-K, stream-K, grid and workspace of a plan whose kernel and tile are
// chosen.  `tuned_sched` and `tuned_splits` are what a tuned entry states
// (0 if none): they apply where the caller leaves the choice to the
// library, and like the automatic choice they never ask for more workspace
// than given.  Under stream-K, a split count (the caller's split_k > 1
// with a forced stream-K schedule, or the tuned one) is the number of K
// slices of each tail tile.
dg_status finish_plan(const dg_gemm_desc *d, Plan p, size_t ws_avail, bool ws_known,
                      int32_t tuned_sched, int32_t tuned_splits, Plan *plan)
{
    const bool forced_sk = d->schedule == DG_SCHED_STREAM_K;
    const bool lib_sched = d->schedule == DG_SCHED_AUTO;
    const bool prefer_sk = lib_sched && tuned_sched == DG_SCHED_STREAM_K;
    const bool forbid_sk = d->schedule == DG_SCHED_DATA_PARALLEL ||
                           (lib_sched && tuned_sched == DG_SCHED_DATA_PARALLEL);
    const int64_t tiles = tiles_of(d, p.tile);
    const int64_t plane = d->batch * d->M * d->N * (int64_t)sizeof(float);
    int32_t slices = 0;      // requested K slices per stream-K tail tile
    if (forced_sk && d->split_k > 1)
        slices = d->split_k;
    else if (prefer_sk && d->split_k == 0 && tuned_splits > 1)
        slices = tuned_splits;
    int32_t S;
    if (!reads_ab(d)) {
        S = 1;
    } else if (forced_sk || (prefer_sk && d->split_k == 0)) {
        S = 1;   // stream-K asked for: no split-K
    } else if (d->split_k >= 1) {
        S = d->split_k;
    } else {
        S = tuned_splits > 0 ? tuned_splits : auto_splits(d, tiles);
        // the automatic choice never asks for more workspace than given
        if (ws_known && S > 1 && (size_t)plane * S > ws_avail)
            S = plane > 0 ? (int32_t)(ws_avail / (size_t)plane) : 1;
        if (S < 2)
            S = 1;
    }
    p.splits = S;
    p.k_per_split = S > 1 ? ceil_div(ceil_div(d->K, S), p.tile.bk) * p.tile.bk : d->K;
    if (p.k_per_split == 0)
        p.k_per_split = 1;
    p.workspace_bytes = S > 1 ? (size_t)plane * S : 0;
    int64_t programs;
    if (__builtin_mul_overflow(tiles, (int64_t)S, &programs) || programs > INT32_MAX ||
        programs * p.tile.threads > (int64_t)UINT32_MAX)
        return DG_ERROR_NOT_SUPPORTED;
    p.programs = programs;
    if (S > 1) {
        int64_t total = d->batch * d->M * d->N;
        int64_t blocks = ceil_div(total, reduce_by_four(d->N, total) ? 1024 : 256);
        p.reduce_blocks = blocks < 65536 ? blocks : 65536;
    }

    // Stream-K ("La GEMM, de zero a cuBLAS", section 2.10: split the work
    // along K so that the last wave is not left mostly idle), for the bf16
    // and fp16 matrix-core kernels on one matrix without split-K.  The tiles of the
    // full waves stay data-parallel; each of the R tail tiles is cut into S
    // K slices, S about wave / R, so the tail fills one more wave.  Only
    // when the tail wave would be less than 85 % full, every slice keeps at
    // least two K steps, and, for the automatic choice, there is at least
    // one full data-parallel wave, K >= 2048 and the caller gives enough
    // workspace for the R * S fp32 partial tiles.  With a shorter K the tail
    // tiles' epilogues cost about as much as their K loop and slicing them
    // gained nothing in measurements (4095 x 4097 x 1000: 101 vs 103 us with
    // GELU, 91 vs 85 us without).  Without a full wave, the partial-tile
    // traffic and the fix-up cost more than the idle compute units: 2048^3
    // ran 41 us sliced against 25 us data-parallel on 128 x 128 tiles, 2048
    // x 2048 x 8192 97 against 72 us.
    const bool sk_possible = (p.kernel == KERNEL_MFMA_BF16 || p.kernel == KERNEL_MFMA_F16) &&
                             d->batch == 1 && S == 1 && reads_ab(d) && p.tile.per_cu > 0;
    if (forced_sk && !sk_possible)
        return DG_ERROR_NOT_SUPPORTED;
    if (sk_possible && !forbid_sk) {
        const int64_t wave = kNumCu * p.tile.per_cu;     // programs resident at once
        const int64_t iters = ceil_div(d->K, p.tile.bk);
        const int64_t dp = tiles / wave * wave;
        const int64_t R = tiles - dp;
        int64_t splits = R > 0 ? wave / R : 0;
        if (splits > iters / 2) splits = iters / 2;
        if (splits > 16) splits = 16;
        if (slices > 0)
            splits = slices < iters ? slices : iters;     // at least one K step each
        const bool want = forced_sk || prefer_sk ||
                          (dp > 0 && R * 100 < wave * 85 && d->K >= 2048);
        if (R > 0 && splits >= 2 && want) {
            StreamK k{};
            k.dp_tiles = dp;
            k.tail_tiles = R;
            k.k_per_split = ceil_div(ceil_div(d->K, splits), p.tile.bk) * p.tile.bk;
            k.tail_splits = ceil_div(d->K, k.k_per_split);   // every slice non-empty
            const size_t ws = (size_t)R * k.tail_splits * p.tile.bm * p.tile.bn * sizeof(float);
            // the automatic choice never asks for more workspace than given
            if (forced_sk || !ws_known || ws <= ws_avail) {
                p.sk = k;
                p.programs = dp + R * k.tail_splits;
                p.workspace_bytes = ws;
                p.fixup_blocks = R * ((int64_t)p.tile.bm * p.tile.bn / 1024);
            }
        }
    }
    *plan = p;
    return DG_SUCCESS;
}


// `key`: the problem to look up in the tuned table (default d).  `keep`:
// without a tuned or forced entry, plan on this tile of the family instead
// of choosing one.
dg_status make_plan(const dg_gemm_desc *d, const void *A, const void *B, size_t ws_avail,
                    bool ws_known, Plan *plan, const dg_gemm_desc *key = nullptr,
                    const TileConfig *keep = nullptr)
{
    Plan p{};
    const int32_t algo = d->algo;
    const TileConfig *table16 = nullptr;   // tiles of the 16-bit matrix-core kernel
    int n16 = 0;
    const TileConfig *table = nullptr;     // tiles of the chosen family
    int ntab = 0;
    if (algo == DG_ALGO_MFMA_BF16 || (algo == DG_ALGO_AUTO && mfma16_eligible(d, DG_BF16, A, B))) {
        if (!mfma16_eligible(d, DG_BF16, A, B))
            return DG_ERROR_NOT_SUPPORTED;
        p.kernel = KERNEL_MFMA_BF16;
        table16 = table = kMfmaBf16Tiles;
        n16 = ntab = kNumMfmaBf16Tiles;
        p.tile = pick_quantised(d, table16, n16);
    } else if (algo == DG_ALGO_MFMA_F16 ||
               (algo == DG_ALGO_AUTO && mfma16_eligible(d, DG_F16, A, B))) {
        if (!mfma16_eligible(d, DG_F16, A, B))
            return DG_ERROR_NOT_SUPPORTED;
        p.kernel = KERNEL_MFMA_F16;
        table16 = table = kMfmaF16Tiles;
        n16 = ntab = kNumMfmaF16Tiles;
        p.tile = pick_quantised(d, table16, n16);
    } else if (algo == DG_ALGO_MFMA_F32 || (algo == DG_ALGO_AUTO && valu_eligible(d, A, B))) {
        // fp32 on the matrix cores: same operand requirements as the VALU kernel
        if (!valu_eligible(d, A, B))
            return DG_ERROR_NOT_SUPPORTED;
        p.kernel = KERNEL_MFMA_F32;
        table = kMfmaF32Tiles;
        ntab = kNumMfmaF32Tiles;
        p.tile = pick_quantised(d, table, ntab);
    } else if (algo == DG_ALGO_VALU_F32) {
        if (!valu_eligible(d, A, B))
            return DG_ERROR_NOT_SUPPORTED;
        p.kernel = KERNEL_VALU_F32;
        table = kValuTiles;
        ntab = kNumValuTiles;
        // The 8 x 16 thread tile (128 x 256 blocks, two resident per CU)
        // when its tiles fill those slots in whole waves (85 % of the last
        // one); otherwise the 8 x 8 tile's smaller blocks (fp32 4096^3:
        // 1532 against 1610 us; 2048^3: 383 against 648 us).
        const TileConfig &narrow = kValuTiles[0], &wide = kValuTiles[1];
        const int64_t slots = 2 * (int64_t)kNumCu;
        const int64_t tiles = tiles_of(d, wide);
        const int64_t waves = ceil_div(tiles, slots);
        const TileConfig *f = forced_tile(table, ntab);
        p.tile = f ? *f : (tiles >= slots && tiles * 100 >= waves * slots * 85) ? wide : narrow;
    } else {
        p.kernel = KERNEL_GENERIC;
        p.tile = kGenericTiles[0];
    }
    // The 16-bit choice above falls back to the small tile when the large
    // one leaves a nearly empty last wave.  When stream-K takes that tail
    // wave instead (automatic choice, workspace given), the large tile with
    // its better flop-per-byte ratio wins: 4352 x 4352 x 8192 (bf16) ran
    // 295 us that way against 415 us on 128 x 128 tiles.
    // An M- or N-contiguous 16-bit operand: only the two tiles of the
    // automatic choice have that variant, and the tuned table was swept on
    // K-contiguous operands, so neither it nor a forced tile applies.
    if (table16 && !k_contiguous(d)) {
        const TileConfig &t256 = table16[0], &t128 = table16[1];
        p.tile = (d->K <= 64 || p.tile.bm != t256.bm || p.tile.bn != t256.bn) ? t128 : t256;
        if (keep)
            p.tile = keep->bm == t256.bm && keep->bn == t256.bn ? t256 : t128;
        Plan done;
        if (p.tile.bm != t256.bm) {
            Plan big = p;
            big.tile = t256;
            if (finish_plan(d, big, ws_avail, ws_known, 0, 0, &done) == DG_SUCCESS &&
                done.sk.tail_tiles > 0 && !keep) {
                *plan = done;
                return DG_SUCCESS;
            }
        }
        return finish_plan(d, p, ws_avail, ws_known, 0, 0, plan);
    }
    const TunedEntry *tuned = nullptr;
    TunedEntry forced;
    if (table && forced_plan(table, ntab, p.kernel, &forced))
        tuned = &forced;
    else if (table && !forced_tile(table, ntab))
        tuned = find_tuned(key ? key : d, p.kernel, table, ntab);
    if (tuned) {
        p.tile = *tile_named(table, ntab, tuned->tile);
        p.tuned = 1;
        return finish_plan(d, p, ws_avail, ws_known, tuned->schedule, tuned->splits, plan);
    }
    if (table && keep) {
        p.tile = *keep;
        return finish_plan(d, p, ws_avail, ws_known, 0, 0, plan);
    }
    if (table16 && !forced_tile(table16, n16) && p.tile.bm != table16[0].bm) {
        Plan big = p;
        big.tile = table16[0];
        Plan done;
        if (finish_plan(d, big, ws_avail, ws_known, 0, 0, &done) == DG_SUCCESS &&
            done.sk.tail_tiles > 0) {
            *plan = done;
            return DG_SUCCESS;
        }
    }
    return finish_plan(d, p, ws_avail, ws_known, 0, 0, plan);
}

// A whole call: the plan of the tiled kernel over columns [0, main.N) and,
// when nrem > 0, the sliver kernel over the last nrem columns.
struct CallPlan {
    dg_gemm_desc main;      // the caller's problem with N cut to the full tile columns
    Plan plan;              // plan of `main`
    int32_t nrem;           // sliver columns (0: none)
};

// The tiled kernels spend a whole tile column on the few columns past the
// last full one and leave their last wave nearly empty: 4095 x 4097 x 1000
// on 128 x 256 tiles is 544 tiles for 512 resident workgroups, and the 32
// tiles of its last column hold one valid column each.  When the library
// chooses the schedule (no split-K or schedule asked for), the plan's tile
// leaves 1 .. kMaxSliver columns past the last full tile column, the full
// columns alone make at least one tile per compute unit and one wave fewer
// than the whole grid (waves of per-CU occupancy x 256 tiles), and A is
// row-major with 16-byte aligned rows, the call runs the tiled plan on the
// full columns and the sliver kernel on the rest.  The full columns' plan
// is looked up in the tuned table under the caller's shape; without an
// entry it keeps the whole grid's tile (re-choosing one for the narrower
// grid took 256 x 256 tiles on the GELU problem: 95 us, against 80 us on
// the 128 x 128 tiles the whole grid chose and 92 us without the split).
// A tuned plan that puts a stream-K tail on the whole grid (the sweep
// timed it against the split) is kept as it is.
dg_status make_call_plan(const dg_gemm_desc *d, const void *A, const void *B, size_t ws_avail,
                         bool ws_known, CallPlan *cp)
{
    cp->main = *d;
    cp->nrem = 0;
    dg_status st = make_plan(d, A, B, ws_avail, ws_known, &cp->plan);
    if (st != DG_SUCCESS)
        return st;
    const Plan &p = cp->plan;
    const bool tiled = p.kernel == KERNEL_MFMA_BF16 || p.kernel == KERNEL_MFMA_F16 ||
                       p.kernel == KERNEL_MFMA_F32;
    if (!tiled || (p.tuned && p.sk.tail_tiles > 0) || d->algo != DG_ALGO_AUTO ||
        d->schedule != DG_SCHED_AUTO || d->split_k != 0 ||
        !reads_ab(d) || d->a_order != DG_ROW_MAJOR ||
        (d->lda * elem_size(d->a_type)) % 16 != 0 ||
        (d->batch > 1 && (d->stride_a * elem_size(d->a_type)) % 16 != 0) ||
        (A && !aligned_to(A, 16)))
        return DG_SUCCESS;     // the sliver kernel reads A's rows in aligned 16-byte pieces
    const int64_t nrem = d->N % p.tile.bn;
    const int64_t n_main = d->N - nrem;
    if (nrem == 0 || nrem > kMaxSliver || n_main < p.tile.bn)
        return DG_SUCCESS;
    // Only where the last tile column costs a wave of its own: the sliver
    // kernel reads all of A once (8 MB on the GELU problem, but 71 MB for
    // 4352 x 4353 x 8192, whose grid keeps its wave count without the column).
    const int64_t rows = ceil_div(d->M, p.tile.bm) * d->batch;
    const int64_t slots = kNumCu * (p.tile.per_cu > 0 ? p.tile.per_cu : 1);
    const int64_t tiles_main = rows * (n_main / p.tile.bn);
    if (tiles_main < kNumCu || ceil_div(tiles_main, slots) == ceil_div(tiles_main + rows, slots))
        return DG_SUCCESS;
    dg_gemm_desc m = *d;
    m.N = n_main;
    Plan pm;
    if (make_plan(&m, A, B, ws_avail, ws_known, &pm, d, p.tuned ? nullptr : &p.tile) != DG_SUCCESS)
        return DG_SUCCESS;           // keep the single plan
    cp->main = m;
    cp->plan = pm;
    cp->nrem = (int32_t)nrem;
    return DG_SUCCESS;
}

void fill_args(const dg_gemm_desc *d, const Plan &p, const void *A, const void *B, void *C,
               void *ws, GemmArgs *g)
{
    memset(g, 0, sizeof *g);
    g->A = A;
    g->B = B;
    g->C = C;
    g->bias = d->bias;
    g->ws = (float *)ws;
    g->M = d->M;
    g->N = d->N;
    g->K = d->K;
    g->lda = d->lda;
    g->ldb = d->ldb;
    g->ldc = d->ldc;
    g->sa = d->stride_a;
    g->sb = d->stride_b;
    g->sc = d->stride_c;
    g->k_per_split = p.k_per_split;
    g->alpha = d->alpha;
    g->beta = d->beta;
    g->a_col = d->a_order == DG_COL_MAJOR;
    g->b_col = d->b_order == DG_COL_MAJOR;
    g->c_col = d->c_order == DG_COL_MAJOR;
    g->c_type = d->c_type;
    g->bias_type = d->bias_type;
    g->act = d->act;
    g->write_partial = p.splits > 1;
    g->ab_type = d->a_type;
    g->sched.num_pid_m = ceil_div(d->M, p.tile.bm);
    g->sched.num_pid_n = ceil_div(d->N, p.tile.bn);
    g->sched.batch = d->batch;
    g->sched.splits = p.splits;
    g->sched.group_m = d->group_m > 0 ? d->group_m : kDefaultGroupM;
    g->sched.xcd_remap = d->xcd_remap >= 0 ? 1 : 0;
    sched_prepare(g->sched);
    g->sk = p.sk;
    g->sk_parts = p.sk.tail_tiles > 0 ? (float *)ws : nullptr;
}

// Enqueue the kernels of a validated call plan on `s`; `ws` is workspace
// of at least cp.plan.workspace_bytes (or null when the plan needs none).
dg_status enqueue(const dg_gemm_desc *d, const CallPlan &cp, const void *A, const void *B,
                  void *C, void *ws, hipStream_t s)
{
    const Plan &p = cp.plan;
    GemmArgs g;
    fill_args(&cp.main, p, A, B, C, ws, &g);
    // One sliver column behind a data-parallel 16-bit plan runs inside the
    // tiled kernel, as workgroups after its tiles: they start as the first
    // tiles finish, within the spread of the tiles' end times, instead of
    // as a separate kernel after the last tile (whose chain of dependent
    // loads took 4.5 to 8 us on its own).
    const bool fused_sliver = cp.nrem == 1 && p.splits == 1 && p.sk.tail_tiles == 0 &&
                              (p.kernel == KERNEL_MFMA_BF16 || p.kernel == KERNEL_MFMA_F16);
    if (fused_sliver) {
        g.sliver_n0 = cp.main.N;
        g.main_programs = p.programs;
        g.sliver_blocks = ceil_div(d->M, kSliverRowsPerBlock);
    }
    hipError_t err = hipSuccess;
    switch (p.kernel) {
    case KERNEL_GENERIC: err = launch_generic(g, p, s); break;
    case KERNEL_VALU_F32: err = launch_valu_f32(g, p, s); break;
    case KERNEL_MFMA_BF16:
    case KERNEL_MFMA_F16: err = launch_mfma16(g, p, s); break;
    case KERNEL_MFMA_F32: err = launch_mfma_f32(g, p, s); break;
    default: return DG_ERROR_NOT_SUPPORTED;
    }
    if (err != hipSuccess)
        return DG_ERROR_LAUNCH;
    if (p.splits > 1) {
        err = launch_splitk_reduce(g, p, s);
        if (err != hipSuccess)
            return DG_ERROR_LAUNCH;
    }
    if (p.sk.tail_tiles > 0) {
        err = launch_streamk_fixup(g, p, s);
        if (err != hipSuccess)
            return DG_ERROR_LAUNCH;
    }
    if (cp.nrem > 0 && !fused_sliver) {
        GemmArgs gs;
        fill_args(d, p, A, B, C, nullptr, &gs);
        err = launch_sliver(gs, cp.main.N, cp.nrem, s);
        if (err != hipSuccess)
            return DG_ERROR_LAUNCH;
    }
    return DG_SUCCESS;
}

// Workspace of dg_gemm_noalloc: one array per GPU, part of the library's
// device code, so it exists from the library's load until the process
// ends and no call allocates.  Host code never uses the array's name as
// an address (on the host it names a stand-in, not device memory): each
// device's own copy is looked up once with hipGetSymbolAddress, with that
// device current, and that pointer is what the kernels receive.
constexpr size_t kScratchBytes = DG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The scratch array of the current device, or null if the runtime fails.
void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

const char *kernel_name(Kernel k)
{
    switch (k) {
    case KERNEL_GENERIC: return "generic";
    case KERNEL_VALU_F32: return "valu_f32";
    case KERNEL_MFMA_BF16: return "mfma_bf16";
    case KERNEL_MFMA_F32: return "mfma_f32";
    case KERNEL_MFMA_F16: return "mfma_f16";
    }
    return "?";
}

} // namespace

extern "C" {

int dg_version(void) { return DG_VERSION; }

const char *dg_status_string(dg_status s)
{
    switch (s) {
    case DG_SUCCESS: return "DG_SUCCESS";
    case DG_ERROR_INVALID_VALUE: return "DG_ERROR_INVALID_VALUE";
    case DG_ERROR_NOT_SUPPORTED: return "DG_ERROR_NOT_SUPPORTED";
    case DG_ERROR_INSUFFICIENT_WORKSPACE: return "DG_ERROR_INSUFFICIENT_WORKSPACE";
    case DG_ERROR_LAUNCH: return "DG_ERROR_LAUNCH";
    }
    return "DG_ERROR_UNKNOWN";
}

dg_status dg_gemm_workspace_size(const dg_gemm_desc *d, size_t *bytes)
{
    if (!bytes)
        return DG_ERROR_INVALID_VALUE;
    Extents e;
    dg_status st = validate_desc(d, &e);
    if (st != DG_SUCCESS)
        return st;
    *bytes = 0;
    if (is_noop(d))
        return DG_SUCCESS;
    CallPlan cp;
    st = make_call_plan(d, nullptr, nullptr, 0, false, &cp);
    if (st != DG_SUCCESS)
        return st;
    *bytes = cp.plan.workspace_bytes;
    return DG_SUCCESS;
}

dg_status dg_gemm_describe(const dg_gemm_desc *d, size_t workspace_bytes, char *buf, size_t len)
{
    if (!buf || len == 0)
        return DG_ERROR_INVALID_VALUE;
    Extents e;
    dg_status st = validate_desc(d, &e);
    if (st != DG_SUCCESS)
        return st;
    if (is_noop(d)) {
        snprintf(buf, len, "noop");
        return DG_SUCCESS;
    }
    CallPlan cp;
    st = make_call_plan(d, nullptr, nullptr, workspace_bytes, true, &cp);
    if (st != DG_SUCCESS)
        return st;
    const Plan &p = cp.plan;
    char sched[128];
    if (p.sk.tail_tiles > 0)
        snprintf(sched, sizeof sched,
                 "stream_k dp_tiles=%lld tail_tiles=%lld tail_splits=%lld tail_k_per_split=%lld",
                 (long long)p.sk.dp_tiles, (long long)p.sk.tail_tiles, (long long)p.sk.tail_splits,
                 (long long)p.sk.k_per_split);
    else
        snprintf(sched, sizeof sched, "data_parallel");
    snprintf(buf, len,
             "kernel=%s tile=%s bm=%d bn=%d bk=%d threads=%d splits=%d k_per_split=%lld "
             "programs=%lld group_m=%d xcd_remap=%d workspace=%zu reduce_blocks=%lld "
             "fixup_blocks=%lld tuned=%d schedule=%s sliver=%d",
             kernel_name(p.kernel), p.tile.name, p.tile.bm, p.tile.bn, p.tile.bk, p.tile.threads,
             p.splits, (long long)p.k_per_split, (long long)p.programs,
             d->group_m > 0 ? d->group_m : kDefaultGroupM, d->xcd_remap >= 0 ? 1 : 0,
             p.workspace_bytes, (long long)p.reduce_blocks, (long long)p.fixup_blocks, p.tuned,
             sched, cp.nrem);
    return DG_SUCCESS;
}

dg_status dg_gemm(const dg_gemm_desc *d, const void *A, const void *B, void *C, void *workspace,
                  size_t workspace_bytes, void *stream)
{
    Extents e;
    dg_status st = validate_desc(d, &e);
    if (st != DG_SUCCESS)
        return st;
    st = validate_ptrs(d, e, A, B, C);
    if (st != DG_SUCCESS)
        return st;
    if (is_noop(d))
        return DG_SUCCESS;
    CallPlan cp;
    st = make_call_plan(d, A, B, workspace ? workspace_bytes : 0, true, &cp);
    if (st != DG_SUCCESS)
        return st;
    if (cp.plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < cp.plan.workspace_bytes)
            return DG_ERROR_INSUFFICIENT_WORKSPACE;
        if (!aligned_to(workspace, 16) ||
            ranges_overlap(workspace, (int64_t)cp.plan.workspace_bytes, C, e.c_bytes))
            return DG_ERROR_INVALID_VALUE;
    }
    return enqueue(d, cp, A, B, C, workspace, (hipStream_t)stream);
}

dg_status dg_gemm_noalloc(const dg_gemm_desc *d, const void *A, const void *B, void *C,
                          void *stream)
{
    Extents e;
    dg_status st = validate_desc(d, &e);
    if (st != DG_SUCCESS)
        return st;
    st = validate_ptrs(d, e, A, B, C);
    if (st != DG_SUCCESS)
        return st;
    if (is_noop(d))
        return DG_SUCCESS;
    // The plan sees the scratch array as the caller's workspace: the
    // automatic choice never asks for more; a forced split-K or stream-K
    // plan that would is refused before any runtime call.
    CallPlan cp;
    st = make_call_plan(d, A, B, kScratchBytes, true, &cp);
    if (st != DG_SUCCESS)
        return st;
    void *ws = nullptr;
    if (cp.plan.workspace_bytes > 0) {
        if (cp.plan.workspace_bytes > kScratchBytes)
            return DG_ERROR_INSUFFICIENT_WORKSPACE;
        ws = scratch_on_current_device();
        if (!ws)
            return DG_ERROR_LAUNCH;
    }
    return enqueue(d, cp, A, B, C, ws, (hipStream_t)stream);
}

dg_status dg_schedule_map(int64_t M, int64_t N, int64_t batch, int32_t split_k, int32_t bm,
                          int32_t bn, int32_t group_m, int32_t xcd_remap, int32_t *out,
                          int64_t out_len)
{
    if (M < 0 || N < 0 || batch < 0 || split_k < 1 || bm < 1 || bn < 1 || group_m < 0 ||
        xcd_remap < -1 || xcd_remap > 1)
        return DG_ERROR_INVALID_VALUE;
    SchedArgs a{};
    a.num_pid_m = ceil_div(M, bm);
    a.num_pid_n = ceil_div(N, bn);
    a.batch = batch;
    a.splits = split_k;
    a.group_m = group_m > 0 ? group_m : kDefaultGroupM;
    a.xcd_remap = xcd_remap >= 0 ? 1 : 0;
    // the decode's arithmetic is 32-bit: no launch has more programs
    int64_t P;
    if (__builtin_mul_overflow(a.num_pid_m, a.num_pid_n, &P) ||
        __builtin_mul_overflow(P, a.batch, &P) || __builtin_mul_overflow(P, (int64_t)a.splits, &P) ||
        P > INT32_MAX)
        return DG_ERROR_NOT_SUPPORTED;
    sched_prepare(a);
    if (P > 0 && (!out || out_len < 4 * P))
        return DG_ERROR_INVALID_VALUE;
    for (int64_t pid = 0; pid < P; ++pid) {
        TileCoord c = decode_program(pid, a);
        out[4 * pid + 0] = (int32_t)c.b;
        out[4 * pid + 1] = c.s;
        out[4 * pid + 2] = c.pid_m;
        out[4 * pid + 3] = c.pid_n;
    }
    return DG_SUCCESS;
}

} // extern "C"
