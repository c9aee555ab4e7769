// Epilogue shared by the matrix-core kernels: a BM x BN tile of fp32
// accumulators held in 32 x 32 (or 16 x 16) MFMA blocks is staged through LDS in chunks
// of rows and stored along C's contiguous dimension in 16-byte runs, with
// alpha, beta * C, bias and the activation applied once per element after
// the K loop ("Skill: Write a Triton GEMM Kernel", Required reasoning
// process step 6), or written raw to the split-K workspace.
#pragma once
#include "common.hpp"

namespace dg {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 16-byte store of a final output or a split-K partial: non-temporal, so
// that the data streams out towards memory instead of staying dirty in the
// L2s until the release at the kernel's end writes it back (the next
// kernel, if any, reads it from beyond the L2s anyway: every kernel starts
// with the L2s invalidated).  Measured: the flat K = 16 problem -6 %, the
// split-K batch -2.5 %, fp32 256^3 in four K slices -7 %.  Stream-K
// partials keep the default policy (0.5 % slower non-temporal on
// 4352 x 4352 x 8192).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
template <bool NT = true>
__device__ __forceinline__ void store16(void *dst, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    if constexpr (NT)
        __builtin_nontemporal_store((u32x4_nt){w0, w1, w2, w3}, (u32x4_nt *)dst);
    else
        *(uint4 *)dst = make_uint4(w0, w1, w2, w3);
}

template <bool NT = true>
__device__ __forceinline__ void store16(void *dst, float v0, float v1, float v2, float v3)
{
    store16<NT>(dst, __float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2),
                __float_as_uint(v3));
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// accesses, not for its global stores.  __syncthreads() also waits for every
// outstanding global store (its release fence covers global memory), which
// would serialise the chunks of the epilogue on HBM write latency; the
// stores read their data from registers at issue, so nothing here needs
// them to have landed.  The memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Epilogue of one run of VEC consecutive outputs along C's contiguous
// dimension: v = act(alpha*acc + beta*C + bias).  `go` is the line (row of
// a row-major C, column of a column-major one), `gi` the first element of
// the run along the line, `lim` the line length; elements past lim are
// left untouched.  `bias_run` points at the staged bias of the run's first
// column.  The branches on beta / bias / act are uniform.
template <int VEC>
__device__ __forceinline__ void run_epilogue(const GemmArgs &g, int64_t b, int64_t go, int64_t gi,
                                             int64_t lim, bool col_major, float (&v)[VEC],
                                             const float *bias_run)
{
    if (g.alpha != 1.0f) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[e] *= g.alpha;
    }
    if (g.beta != 0.0f) {
        const int64_t base = b * g.sc + go * g.ldc + gi;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (gi + e < lim)
                v[e] = fmaf(g.beta, load_as_f32(g.C, g.c_type, base + e), v[e]);
    }
    if (g.bias) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[e] += col_major ? bias_run[0] : bias_run[e];
    }
    if (g.act != ACT_NONE)
        activate_n<VEC>(v, g.act);
}

// Store rows [r0, r0 + ROWS) of a BM x BN output tile from an LDS chunk
// (fp32, row-major, row stride LD) to C of dtype OUT.  The NT threads walk
// C's contiguous dimension in runs of VEC elements (16 bytes: 8 16-bit or
// 4 fp32 values); a run inside the matrix and 16-byte aligned is written
// with one vector store, otherwise element by element (ragged edges, odd
// ldc).  Serves column-major C (row-major C takes tile_epilogue_rows).
template <int OUT, int ROWS, int BN, int LD, int NT>
__device__ __forceinline__ void store_chunk(const GemmArgs &g, const TileCoord &tc,
                                            const float *chunk, int64_t m0, int64_t n0, int r0,
                                            const float *bias_s)
{
    constexpr int VEC = OUT == DT_F32 ? 4 : 8;
    const bool col_major = g.c_col;
    const int64_t ld = g.ldc;
    const int64_t base = tc.b * g.sc;
    // runs per line: along n (row-major) or along m (column-major)
    const int line_len = col_major ? ROWS : BN;
    const int runs_per_line = line_len / VEC;
    const int nruns = ROWS * BN / VEC;
    const int64_t inner_lim = col_major ? g.M : g.N;
    const int64_t outer_lim = col_major ? g.N : g.M;
    for (int r = threadIdx.x; r < nruns; r += NT) {
        const int line = r / runs_per_line;
        const int first = (r % runs_per_line) * VEC;
        // tile-relative coordinates of the run's first element
        const int row = col_major ? r0 + first : r0 + line;
        const int col = col_major ? line : first;
        const int64_t go = col_major ? n0 + col : m0 + row;   // line index in C
        const int64_t gi = col_major ? m0 + row : n0 + col;   // position along the line
        if (go >= outer_lim || gi >= inner_lim)
            continue;
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[e] = col_major ? chunk[(row - r0 + e) * LD + col] : chunk[(row - r0) * LD + col + e];
        run_epilogue<VEC>(g, tc.b, go, gi, inner_lim, col_major, v, bias_s + col);
        const int64_t off = base + go * ld + gi;
        const bool full = gi + VEC <= inner_lim;
        if (OUT == DT_F32) {
            float *dst = (float *)g.C + off;
            if (full && ((uintptr_t)dst & 15) == 0) {
                store16(dst, v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (gi + e < inner_lim)
                        dst[e] = v[e];
            }
        } else {
            uint16_t *dst = (uint16_t *)g.C + off;
            uint16_t h[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                h[e] = f32_to_half<OUT>(v[e]);
            if (full && ((uintptr_t)dst & 15) == 0) {
                uint32_t w[VEC / 2];
#pragma unroll
                for (int e = 0; e < VEC / 2; ++e)
                    w[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
                store16(dst, w[0], w[1], w[2], w[3]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (gi + e < inner_lim)
                        dst[e] = h[e];
            }
        }
    }
}

// LDS bytes tile_epilogue needs for a tile BN columns wide, for
// accumulators in MS x MS MFMA blocks.  A staged row is BN + 8 floats for
// 32 x 32 blocks: the two 32-lane halves of a wave's accumulator write, 4
// rows apart, then fall on disjoint halves of the 64 banks.  For 16 x 16
// blocks it is BN + 20: the four 16-lane groups, 4 rows apart, fall on four
// disjoint quarters.  Rows stay 16-byte aligned either way.
constexpr int kEpilogueRows = 64;
constexpr int epilogue_ld(int BN, int MS = 32) { return MS == 32 ? BN + 8 : BN + 20; }
constexpr int epilogue_lds_bytes(int BN, int MS = 32)
{
    return (kEpilogueRows * epilogue_ld(BN, MS) + BN) * 4;
}

// Block shape of an accumulator argument (a view type of 16 x 16 blocks
// specialises it).
template <typename ACC> struct acc_traits { static constexpr int MS = 32; };

// A wave's FM x FN 16 x 16 accumulator blocks (v_mfma_f32_16x16x32_*), as
// the epilogue takes them: it stages block (i, j) value v of lane 16 g + c
// at row 16 i + 4 g + v, column 16 j + c of the wave tile.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int FM, int FN>
struct Acc16View {
    const f32x4_t (&a)[FM][FN];
};
template <int FM, int FN> struct acc_traits<Acc16View<FM, FN>> { static constexpr int MS = 16; };

template <int FM, int FN>
__device__ __forceinline__ const f32x4_t &acc_block16(const Acc16View<FM, FN> &v, int i, int j)
{
    return v.a[i][j];
}

// The epilogue reads a wave's accumulators one block at a time: FM x FN
// 32 x 32 blocks in the 32 x 32 MFMA register layout through acc_block, or,
// for an Acc16View (acc_traits MS = 16), 2FM x 2FN 16 x 16 blocks through
// acc_block16, each staged in its own layout.
template <int FM, int FN>
__device__ __forceinline__ const f32x16_t &acc_block(const f32x16_t (&acc)[FM][FN], int i, int j)
{
    return acc[i][j];
}

// Accumulator blocks of rows [c * EP_ROWS, (c + 1) * EP_ROWS) of the tile into
// the LDS chunk (fp32, row stride EP_LD).  Lane l's value v of a 32 x 32
// block is row 8*(v/4) + 4*(l/32) + v%4, column l%32 of that block; wave
// (wm, wn) owns blocks FM x FN at rows wm*TM + 32i, columns wn*TN + 32j
// (16 x 16 blocks: see Acc16View).
// Tile row r is stored shifted right by shift(r) < 8 floats (0 for the
// generic path), with EP_LD leaving room for it.
template <int BM, int BN, int WM, int WN, typename Shift, typename ACC>
__device__ __forceinline__ void stage_chunk(float *chunk, int c, const ACC &acc, Shift shift)
{
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int AMS = acc_traits<ACC>::MS;
    constexpr int EP_ROWS = kEpilogueRows, EP_LD = epilogue_ld(BN, AMS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int frag_half = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int row0 = wm * TM + i * 32 - c * EP_ROWS;   // block's first row in the chunk
        if (row0 >= 0 && row0 < EP_ROWS) {
            if constexpr (AMS == 32) {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const f32x16_t &blk = acc_block(acc, i, j);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = row0 + 8 * (v / 4) + 4 * frag_half + (v % 4);
                        chunk[row * EP_LD + shift(c * EP_ROWS + row) + wn * TN + (lane & 31) +
                              j * 32] = blk[v];
                    }
                }
            } else {
                // 16 x 16 blocks 2i, 2i + 1: lane 16 g + c holds rows
                // 4 g .. 4 g + 3 of column c
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int j = 0; j < 2 * FN; ++j) {
                        const auto &blk = acc_block16(acc, 2 * i + bi, j);
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int row = row0 + 16 * bi + 4 * (lane >> 4) + v;
                            chunk[row * EP_LD + shift(c * EP_ROWS + row) + wn * TN + (lane & 15) +
                                  j * 16] = blk[v];
                        }
                    }
            }
        }
    }
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Epilogue of a whole tile (all BM x BN outputs inside the output): the
// interior case of tile_epilogue_rows, with its arithmetic and stores, minus
// the per-run bounds logic.  Chunk c holds block row c of every wave's
// accumulators (32 * WM tile rows, so all waves stage each chunk).  Thread
// t owns one column slot js = t mod RPR and the rows t / RPR + q * (NT / RPR)
// of each chunk.  The runs are taken in groups whose values fit the
// registers left beside the accumulators (REGS per lane in all, the budget
// the kernel was compiled to): all of a group's LDS reads (and C reads when
// beta != 0) are issued before its first store, so their latencies overlap
// instead of adding up run after run.
//
// Without SHIFTED every row starts on a 16-byte boundary and slot js is the
// row's 16-byte block js.  With SHIFTED, row r starts s(r) = (d0 + r * dl)
// mod VEC elements past a boundary and is staged shifted right by s(r), so
// each 16-byte block of the output row is one aligned vector of the staged
// row.  A row with s > 0 has a partial head block, RPR - 1 full blocks and
// a partial tail block: slot js takes full block js + 1 (the last slot has
// none), and a pass per chunk stores the head and tail elements one by one.
template <int BM, int BN, int WM, int WN, bool PARTIAL, int OUT, int REGS, bool SHIFTED,
          bool STREAM = true, typename ACC>
__device__ __forceinline__ void tile_epilogue_whole(const GemmArgs &g, char *out, int64_t ld,
                                                    int64_t n0, float *lds, int d0, int dl,
                                                    const ACC &acc)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int CH_ROWS = 32 * WM;                  // tile rows per chunk
    constexpr int AMS = acc_traits<ACC>::MS;
    constexpr int EP_LD = epilogue_ld(BN, AMS);
    constexpr bool HALF_OUT = OUT != DT_F32;
    constexpr int VEC = HALF_OUT ? 8 : 4;             // outputs per 16-byte block
    constexpr int ES = HALF_OUT ? 2 : 4;              // output element size
    constexpr int RPR = BN / VEC;                     // column slots (full blocks of an aligned row)
    constexpr int RSTEP = NT / RPR;                   // chunk rows between a thread's runs
    constexpr int RUNS = CH_ROWS / RSTEP;             // runs per thread per chunk
    constexpr int EDGE = CH_ROWS * 2 * VEC / NT;      // head / tail elements per thread per chunk
    static_assert(CH_ROWS <= kEpilogueRows, "chunk fits the staging buffer");
    static_assert(NT % RPR == 0 && 32 % RSTEP == 0 && RUNS * RSTEP == CH_ROWS, "run split");
    static_assert(EDGE * NT == CH_ROWS * 2 * VEC, "edge split");
    static_assert(EP_LD >= BN + VEC, "room for the row shift and the tail block");
    // registers per run in flight (values, and C's when beta != 0); about
    // 40 more stay with addresses, bias and loop state
    constexpr int PER_RUN = VEC + (PARTIAL ? 0 : 4);
    constexpr int SPARE = REGS - BM * BN / NT - 40;
    constexpr int GROUP = PER_RUN * RUNS <= SPARE ? RUNS
                        : PER_RUN * (RUNS / 2) <= SPARE ? RUNS / 2
                        : PER_RUN * (RUNS / 4) <= SPARE ? RUNS / 4 : 1;
    static_assert(RUNS % GROUP == 0, "groups split the runs");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int frag_half = lane >> 5;
    const int js = tid % RPR;                         // column slot
    const int rt = tid / RPR;                         // first chunk row of the thread
    const int64_t ld_bytes = ld * ES;
    char *rowbase = out + (int64_t)rt * ld_bytes;
    const float *rdrow = lds + rt * EP_LD;
    float *bias_s = lds + kEpilogueRows * EP_LD;      // SHIFTED: the tile's bias
    // misalignment (elements) of tile row r
    auto shift = [&](int r) { return SHIFTED ? (d0 + r * dl) & (VEC - 1) : 0; };
    // chunk row cr of chunk c is tile row (cr / 32) * TM + c * 32 + cr % 32
    auto tile_row = [&](int c, int cr) { return (cr / 32) * TM + c * 32 + cr % 32; };
    // Every run of a thread is at tile row rt plus a multiple of 8 (32-row
    // blocks, TM-row wave blocks and RSTEP-row steps are all multiples of
    // VEC), so with the row misalignment stepping by dl per row, all of them
    // share one shift, one block slot and so one set of VEC columns: the
    // thread's bias values are read once, into registers.
    const int sh_t = shift(rt);
    const int col_t = (js + (sh_t != 0 ? 1 : 0)) * VEC - sh_t;   // first column of the runs
    float bias[VEC];
    const bool has_bias = !PARTIAL && g.bias;
    if (has_bias) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            bias[e] = col_t + e < BN ? load_as_f32(g.bias, g.bias_type, n0 + col_t + e) : 0.0f;
        if (SHIFTED) {
            // the head and tail elements, one by one
            for (int t = tid; t < BN; t += NT)
                bias_s[t] = load_as_f32(g.bias, g.bias_type, n0 + t);
        }
    }
    const bool read_c = !PARTIAL && g.beta != 0.0f;
    // Block row I of the wave's accumulators -> chunk rows wm * 32 + [0, 32),
    // each shifted by its tile row's misalignment.
    auto stage = [&](auto I) {
        if constexpr (AMS == 32) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const f32x16_t &blk = acc_block(acc, decltype(I)::value, j);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rb = 8 * (v / 4) + 4 * frag_half + (v % 4);
                    lds[(wm * 32 + rb) * EP_LD + shift(wm * TM + decltype(I)::value * 32 + rb) +
                        wn * TN + (lane & 31) + j * 32] = blk[v];
                }
            }
        } else {
            // 16 x 16 blocks 2I, 2I + 1: lane 16 g + c holds rows 4 g .. 4 g + 3
            // of column c
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int j = 0; j < 2 * FN; ++j) {
                    const auto &blk = acc_block16(acc, 2 * decltype(I)::value + bi, j);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int rb = 16 * bi + 4 * (lane >> 4) + v;
                        lds[(wm * 32 + rb) * EP_LD + shift(wm * TM + decltype(I)::value * 32 + rb) +
                            wn * TN + (lane & 15) + j * 16] = blk[v];
                    }
                }
        }
    };
    // alpha, beta * C, bias and activation of one value at tile column col
    // (the edge elements; the runs apply the same steps group-wide).
    auto finish_one = [&](float v, const char *cptr, int col) {
        if (PARTIAL)
            return v;
        v *= g.alpha;
        if (read_c)
            v = fmaf(g.beta, HALF_OUT ? half_to_f32<OUT>(*(const uint16_t *)cptr) : *(const float *)cptr, v);
        if (has_bias)
            v += bias_s[col];
        return activate(v, g.act);
    };
    // One copy of the chunk code per chunk, each with its chunk index a
    // constant: a loop over the chunks, unrolled or not, leaves the
    // accumulators indexed at run time (and so in scratch memory) once its
    // body - the unrolled runs and their activations - is large.
    static_for<FM>([&](auto I) {
        constexpr int c = decltype(I)::value;
        stage(I);
        lds_barrier();
        static_for<RUNS / GROUP>([&](auto G) {
            constexpr int q0 = decltype(G)::value * GROUP;
            // run u: chunk row rt + q * RSTEP, tile row trow[u] (relative to
            // row rt), 16-byte block at tile column col[u]; full[u] is false
            // for the last slot of a shifted row, which has no full block
            int trow[GROUP], blk[GROUP], col[GROUP];
            bool full[GROUP];
#pragma unroll
            for (int u = 0; u < GROUP; ++u) {
                const int q = q0 + u;
                trow[u] = tile_row(c, q * RSTEP);
                const int sh = shift(trow[u] + rt);
                blk[u] = js + (sh != 0 ? 1 : 0);
                col[u] = blk[u] * VEC - sh;
                full[u] = !SHIFTED || sh == 0 || js < RPR - 1;
            }
            uint4 cin[GROUP];
            if (read_c) {
#pragma unroll
                for (int u = 0; u < GROUP; ++u)
                    if (full[u])
                        cin[u] = *(const uint4 *)(rowbase + (int64_t)trow[u] * ld_bytes + (int64_t)col[u] * ES);
            }
            // A 16-bit output's run is 8 staged floats, two 16-byte halves
            // 32 bytes apart from the next slot's: slots j and j + 8 would
            // share bank groups.  Slots with bit 3 set read their halves in
            // the other order, so the 16 lanes of one read cover all 16
            // groups.
            float v[GROUP][VEC];
            const bool swap_halves = VEC == 8 && ((js >> 3) & 1);
#pragma unroll
            for (int u = 0; u < GROUP; ++u) {
                const float *rp = &rdrow[(q0 + u) * RSTEP * EP_LD + blk[u] * VEC];
                if constexpr (VEC == 8) {
                    const float4 x0 = *(const float4 *)(rp + (swap_halves ? 4 : 0));
                    const float4 x1 = *(const float4 *)(rp + (swap_halves ? 0 : 4));
                    const float4 lo = swap_halves ? x1 : x0, hi = swap_halves ? x0 : x1;
                    v[u][0] = lo.x; v[u][1] = lo.y; v[u][2] = lo.z; v[u][3] = lo.w;
                    v[u][4] = hi.x; v[u][5] = hi.y; v[u][6] = hi.z; v[u][7] = hi.w;
                } else {
                    const float4 x = *(const float4 *)rp;
                    v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
                }
            }
            // Each step covers the whole group, so every uniform branch
            // (beta, bias, activation) is taken once per group, not per run.
            if (!PARTIAL) {
                if (g.alpha != 1.0f) {
#pragma unroll
                    for (int u = 0; u < GROUP; ++u)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            v[u][e] *= g.alpha;
                }
                if (read_c) {
#pragma unroll
                    for (int u = 0; u < GROUP; ++u) {
                        const uint32_t w[4] = {cin[u].x, cin[u].y, cin[u].z, cin[u].w};
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const float x = HALF_OUT ? half_to_f32<OUT>((uint16_t)(w[e / 2] >> (16 * (e % 2))))
                                                     : __uint_as_float(w[e]);
                            v[u][e] = fmaf(g.beta, x, v[u][e]);
                        }
                    }
                }
                if (has_bias) {
#pragma unroll
                    for (int u = 0; u < GROUP; ++u)
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            v[u][e] += bias[e];
                }
                auto act_all = [&](auto A) {
#pragma unroll
                    for (int u = 0; u < GROUP; ++u)
                        activate_n<decltype(A)::value, VEC>(v[u]);
                };
                if (g.act == ACT_GELU_ERF)
                    act_all(std::integral_constant<int32_t, ACT_GELU_ERF>{});
                else if (g.act == ACT_GELU_TANH)
                    act_all(std::integral_constant<int32_t, ACT_GELU_TANH>{});
            }
#pragma unroll
            for (int u = 0; u < GROUP; ++u) {
                if (!full[u])
                    continue;
                char *dst = rowbase + (int64_t)trow[u] * ld_bytes + (int64_t)col[u] * ES;
                if (HALF_OUT) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (uint32_t)f32_to_half<OUT>(v[u][2 * e]) |
                               ((uint32_t)f32_to_half<OUT>(v[u][2 * e + 1]) << 16);
                    store16<STREAM>(dst, w[0], w[1], w[2], w[3]);
                } else {
                    store16<STREAM>(dst, v[u][0], v[u][1], v[u][2], v[u][3]);
                }
            }
        });
        if constexpr (SHIFTED) {
            // head block (elements s .. VEC-1 at tile columns 0 .. VEC-s-1)
            // and tail block (elements 0 .. s-1 at tile columns BN-s .. BN-1)
            // of every shifted chunk row, EDGE elements per thread
#pragma unroll
            for (int i = 0; i < EDGE; ++i) {
                const int slot = tid * EDGE + i;
                const int cr = slot / (2 * VEC), k = slot % (2 * VEC);
                const int tr = tile_row(c, cr);
                const int sh = shift(tr);
                const bool head = k < VEC;
                const int e = head ? k : k - VEC;
                if (sh == 0 || (head ? e < sh : e >= sh))
                    continue;
                const int tc = head ? e - sh : BN - sh + e;
                char *dst = out + (int64_t)tr * ld_bytes + (int64_t)tc * ES;
                const float v = finish_one(lds[cr * EP_LD + (head ? 0 : BN) + e], dst, tc);
                if (HALF_OUT)
                    *(uint16_t *)dst = f32_to_half<OUT>(v);
                else
                    *(float *)dst = v;
            }
        }
        lds_barrier();
    });
}

// Epilogue of a tile of a row-major output (C, or the split-K workspace
// when PARTIAL, fp32), of dtype OUT, at any alignment and with ragged
// edges.  Each output row is cut into 16-byte aligned runs of VEC elements
// (8 16-bit or 4 fp32 values) at
// its own alignment: a row whose first element sits delta elements past a
// 16-byte boundary has a partial head run, BN / VEC - 1 full runs and a
// partial tail.  The row is staged shifted by delta in LDS, so every run
// reads one aligned 16-byte vector; full runs are written with one 16-byte
// store (and read C with one 16-byte load when beta != 0), partial runs and
// runs cut by the matrix edge element by element.
// `out` points at the tile's first element, `ld` is the output's row
// stride (elements), rows x cols the part of the tile inside the output and
// n0 the tile's first column (for the bias).
template <int BM, int BN, int WM, int WN, bool PARTIAL, int OUT, int REGS = 512,
          bool STREAM = true, typename ACC>
__device__ __forceinline__ void tile_epilogue_rows(const GemmArgs &g, char *out, int64_t ld,
                                                   int rows, int cols, int64_t n0, float *lds,
                                                   const ACC &acc)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int EP_ROWS = kEpilogueRows, EP_LD = epilogue_ld(BN, acc_traits<ACC>::MS);
    static_assert(!PARTIAL || OUT == DT_F32, "partials are fp32");
    constexpr bool HALF_OUT = OUT != DT_F32;
    constexpr int VEC = HALF_OUT ? 8 : 4;             // outputs per 16-byte run
    constexpr int RPR = BN / VEC + 1;                 // runs per row (head + full + tail)
    constexpr int ES = HALF_OUT ? 2 : 4;              // output element size
    static_assert(EP_LD >= BN + VEC - 1, "room for the row shift");
    const int tid = threadIdx.x;
    float *chunk = lds;
    float *bias_s = chunk + EP_ROWS * EP_LD;
    const int64_t ld_bytes = ld * ES;
    // misalignment (elements) of tile row r: (d0 + r * dl) mod VEC
    const int d0 = (int)(((uintptr_t)out % 16) / ES);
    const int dl = (int)(ld % VEC);
    auto shift = [&](int r) { return (d0 + r * dl) & (VEC - 1); };
    if (rows == BM && cols == BN) {
        if (d0 == 0 && dl == 0)
            tile_epilogue_whole<BM, BN, WM, WN, PARTIAL, OUT, REGS, false, STREAM>(g, out, ld, n0, lds, 0, 0,
                                                                           acc);
        else
            tile_epilogue_whole<BM, BN, WM, WN, PARTIAL, OUT, REGS, true, STREAM>(g, out, ld, n0, lds, d0, dl,
                                                                          acc);
        return;
    }
    const bool has_bias = !PARTIAL && g.bias;
    if (has_bias) {
        for (int t = tid; t < BN; t += NT)
            bias_s[t] = t < cols ? load_as_f32(g.bias, g.bias_type, n0 + t) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < BM / EP_ROWS; ++c) {
        stage_chunk<BM, BN, WM, WN>(chunk, c, acc, shift);
        lds_barrier();
        for (int r = tid; r < EP_ROWS * RPR; r += NT) {
            const int row = r / RPR, j = r % RPR;
            const int trow = c * EP_ROWS + row;                // tile row
            const int c0 = j * VEC - shift(trow);              // tile column of element 0
            const int lo = c0 < 0 ? -c0 : 0;
            const int hi = cols - c0 < VEC ? cols - c0 : VEC;
            if (trow >= rows || lo >= hi)
                continue;
            const bool full = lo == 0 && hi == VEC;
            float v[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const float4 q = *(const float4 *)&chunk[row * EP_LD + j * VEC + e];
                v[e] = q.x; v[e + 1] = q.y; v[e + 2] = q.z; v[e + 3] = q.w;
            }
            char *dst = out + (int64_t)trow * ld_bytes + (int64_t)c0 * ES;   // 16-byte aligned
            if (!PARTIAL) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    v[e] *= g.alpha;
                if (g.beta != 0.0f) {
                    if (full) {
                        const uint4 cin = *(const uint4 *)dst;
                        const uint32_t w[4] = {cin.x, cin.y, cin.z, cin.w};
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const float x = HALF_OUT ? half_to_f32<OUT>((uint16_t)(w[e / 2] >> (16 * (e % 2))))
                                                     : __uint_as_float(w[e]);
                            v[e] = fmaf(g.beta, x, v[e]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            if (e >= lo && e < hi) {
                                const float x = HALF_OUT ? half_to_f32<OUT>(((const uint16_t *)dst)[e])
                                                         : ((const float *)dst)[e];
                                v[e] = fmaf(g.beta, x, v[e]);
                            }
                        }
                    }
                }
                if (has_bias) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const int col = c0 + e;
                        v[e] += bias_s[col < 0 ? 0 : (col < BN ? col : BN - 1)];
                    }
                }
                if (g.act != ACT_NONE)
                    activate_n<VEC>(v, g.act);
            }
            if (HALF_OUT) {
                uint16_t h[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    h[e] = f32_to_half<OUT>(v[e]);
                if (full) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
                    store16<STREAM>(dst, w[0], w[1], w[2], w[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (e >= lo && e < hi)
                            ((uint16_t *)dst)[e] = h[e];
                }
            } else {
                if (full) {
                    store16<STREAM>(dst, v[0], v[1], v[2], v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (e >= lo && e < hi)
                            ((float *)dst)[e] = v[e];
                }
            }
        }
        lds_barrier();
    }
}

// Stage and store the whole tile.  `lds` must hold epilogue_lds_bytes(BN)
// bytes and no wave may still be reading it for other purposes.  Row-major
// outputs (and split-K partials) take tile_epilogue_rows; a column-major C
// goes through store_chunk.
template <int BM, int BN, int WM, int WN, int REGS = 512, typename ACC>
__device__ __forceinline__ void tile_epilogue(const GemmArgs &g, const TileCoord &tc, float *lds,
                                              int64_t m0, int64_t n0, const ACC &acc)
{
    const int rows = (int)(g.M - m0 < BM ? g.M - m0 : BM);
    const int cols = (int)(g.N - n0 < BN ? g.N - n0 : BN);
    if (g.write_partial) {
        float *out = g.ws + (((int64_t)tc.s * g.sched.batch + tc.b) * g.M + m0) * g.N + n0;
        tile_epilogue_rows<BM, BN, WM, WN, true, DT_F32, REGS>(g, (char *)out, g.N, rows, cols, n0,
                                                         lds, acc);
        return;
    }
    if (!g.c_col) {
        if (g.c_type == DT_F32) {
            char *out = (char *)g.C + (tc.b * g.sc + m0 * g.ldc + n0) * 4;
            tile_epilogue_rows<BM, BN, WM, WN, false, DT_F32, REGS>(g, out, g.ldc, rows, cols, n0, lds,
                                                              acc);
        } else {
            char *out = (char *)g.C + (tc.b * g.sc + m0 * g.ldc + n0) * 2;
            if (g.c_type == DT_BF16)
                tile_epilogue_rows<BM, BN, WM, WN, false, DT_BF16, REGS>(g, out, g.ldc, rows, cols, n0,
                                                                   lds, acc);
            else
                tile_epilogue_rows<BM, BN, WM, WN, false, DT_F16, REGS>(g, out, g.ldc, rows, cols, n0,
                                                                  lds, acc);
        }
        return;
    }
    constexpr int NT = 64 * WM * WN;
    constexpr int EP_ROWS = kEpilogueRows;
    constexpr int EP_LD = epilogue_ld(BN, acc_traits<ACC>::MS);
    const int tid = threadIdx.x;
    float *chunk = lds;
    // the tile's BN bias values, read from global memory once
    float *bias_s = chunk + EP_ROWS * EP_LD;
    if (g.bias) {
        for (int t = tid; t < BN; t += NT)
            bias_s[t] = n0 + t < g.N ? load_as_f32(g.bias, g.bias_type, n0 + t) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < BM / EP_ROWS; ++c) {
        stage_chunk<BM, BN, WM, WN>(chunk, c, acc, [](int) { return 0; });
        lds_barrier();
        if (g.c_type == DT_BF16)
            store_chunk<DT_BF16, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS, bias_s);
        else if (g.c_type == DT_F16)
            store_chunk<DT_F16, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS, bias_s);
        else
            store_chunk<DT_F32, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS, bias_s);
        lds_barrier();
    }
}

} // namespace dg
