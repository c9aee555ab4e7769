// bf16 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation.
//
// The structure is the tiled blocked GEMM of "GEMM Kernel Optimization"
// (Core Technique: one workgroup per BM x BN output tile, K walked in
// BK chunks, fp32 accumulators, cast on store) with the matrix-core
// inner loop of its "Tensor Core Utilization" section and the three tiling
// levels of "La GEMM, de zero a cuBLAS" (workgroup tile in LDS, wave tile
// in registers, 32 x 32 x 16 MFMA fragments).
//
// Operands: A row-major (M x K) and B column-major (K x N), i.e. both with
// K contiguous, which is the order an MFMA lane consumes: lane l supplies 8
// consecutive k of row (l mod 32) of A and of column (l mod 32) of B.
//
// Data path per K tile (BK = 64):
//   global -> registers: 16-byte loads, 8 consecutive threads cover one
//     128-byte row of the tile (coalesced), masked on the row bound and the
//     split's K range with zero fill;
//   registers -> LDS: row r's 16-byte chunk c is stored at chunk position
//     c ^ ((r / 2) mod 8) (XOR swizzle).  LDS serves a 128-bit access 16
//     lanes at a time across 256 bytes of banks; 16 lanes reading 16
//     consecutive rows at one logical chunk, or 16 lanes writing two
//     consecutive rows, then touch 16 different 16-byte bank groups;
//   LDS -> registers: ds_read_b128 fragments, 4 k-steps of 16 per tile;
//   MFMA: each wavefront owns a TM x TN wave tile = FM x FN blocks of
//     32 x 32, accumulated in FM*FN*16 fp32 registers per lane.
// The next tile is fetched into registers while the current one is
// multiplied, then written to the other LDS buffer: two LDS stages, one
// barrier per K tile ("La GEMM, de zero a cuBLAS", section 2.8).
//
// Requirements checked on the host: bf16 A (row-major) and B (column-
// major); 16-byte aligned base pointers; lda, ldb and the batch strides
// multiples of 8 elements.  K may be anything (the last chunk is masked
// element by element).
#include "launch.hpp"

namespace dg {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int MBK = 64;   // K per LDS tile: 8 chunks of 8 bf16 per row

// 8 bf16 of one row at k = k_first .. k_first+7, zero for k >= ke (the
// K-boundary mask of the last, partial K tile).  `row` points at k = 0 of
// the row; ke >= 1.  Branch-free: the index is clamped to ke-1, so every
// load stays inside the row, and masked elements are replaced by 0.
__device__ __forceinline__ uint4 load_chunk_tail(const uint16_t *row, int64_t k_first,
                                                 int64_t ke)
{
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = k_first + j;
        const uint32_t v = row[k < ke ? k : ke - 1];
        w[j / 2] |= (k < ke ? v : 0u) << (16 * (j % 2));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Epilogue of one run of VEC consecutive outputs along C's contiguous
// dimension: v = act(alpha*acc + beta*C + bias).  `go` is the line (row of
// a row-major C, column of a column-major one), `gi` the first element of
// the run along the line, `lim` the line length; elements past lim are
// left untouched.  The branches on beta / bias / act are uniform.
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
#pragma unroll
    for (int e = 0; e < VEC; ++e)
        v[e] *= g.alpha;
    if (g.beta != 0.0f) {
        const int64_t base = b * g.sc + go * g.ldc + gi;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (gi + e < lim)
                v[e] = fmaf(g.beta, load_as_f32(g.C, g.c_bf16, base + e), v[e]);
    }
    if (g.bias) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[e] += col_major ? bias_run[0] : bias_run[e];
    }
    if (g.act != ACT_NONE) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            v[e] = activate(v[e], g.act);
    }
}

// Store rows [r0, r0 + ROWS) of a BM x BN output tile from an LDS chunk
// (fp32, row-major, row stride LD) to C, or when PARTIAL to the split-K
// workspace ([split][batch][M][N], row-major).  The NT threads walk C's
// contiguous dimension in runs of VEC elements (16 bytes: 8 bf16 or 4
// fp32); a run inside the matrix and 16-byte aligned is written with one
// vector store, otherwise element by element (ragged edges, odd ldc).
template <int VEC, bool PARTIAL, bool BF16_OUT, int ROWS, int BN, int LD, int NT>
__device__ __forceinline__ void store_chunk(const GemmArgs &g, const TileCoord &tc,
                                            const float *chunk, int64_t m0, int64_t n0, int r0,
                                            const float *bias_s)
{
    const bool col_major = !PARTIAL && g.c_col;
    const int64_t ld = PARTIAL ? g.N : g.ldc;
    const int64_t base = PARTIAL ? ((int64_t)tc.s * g.sched.batch + tc.b) * g.M * g.N
                                 : tc.b * g.sc;
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
        if (!PARTIAL)
            run_epilogue<VEC>(g, tc.b, go, gi, inner_lim, col_major, v,
                              bias_s + col);
        const int64_t off = base + go * ld + gi;
        const bool full = gi + VEC <= inner_lim;
        if (PARTIAL || !BF16_OUT) {
            float *dst = (PARTIAL ? g.ws : (float *)g.C) + off;
            if (full && ((uintptr_t)dst & 15) == 0) {
                *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
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
                h[e] = f32_to_bf16(v[e]);
            if (full && ((uintptr_t)dst & 15) == 0) {
                uint32_t w[VEC / 2];
#pragma unroll
                for (int e = 0; e < VEC / 2; ++e)
                    w[e] = (uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16);
                *(uint4 *)dst = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (gi + e < inner_lim)
                        dst[e] = h[e];
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_bf16_kernel(GemmArgs g)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;    // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 blocks per wave
    constexpr int ROWS_PER_PASS = NT / 8;        // tile rows loaded per pass
    constexpr int ACH = BM / ROWS_PER_PASS;      // 16-byte chunks per thread (A)
    constexpr int BCH = BN / ROWS_PER_PASS;      // (B)
    constexpr int A_STAGE = BM * 8, B_STAGE = BN * 8;   // uint4 per stage
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load split");

    extern __shared__ uint4 lds[];
    uint4 *As = lds;                  // [2][BM rows][8 chunks]
    uint4 *Bs = lds + 2 * A_STAGE;    // [2][BN cols][8 chunks]

    const TileCoord tc = decode_program(blockIdx.x, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * BM;
    const int64_t n0 = (int64_t)tc.pid_n * BN;
    int64_t kb, ke;
    split_range(g, tc.s, kb, ke);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int kc = tid & 7;          // chunk column this thread loads
    const int r0 = tid >> 3;         // first tile row this thread loads
    const uint16_t *A = (const uint16_t *)g.A + tc.b * g.sa;
    const uint16_t *B = (const uint16_t *)g.B + tc.b * g.sb;
    const int64_t M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    // Per-thread source pointers of the rows this thread loads.  Rows past
    // M (or N) are clamped to the last row: the loads stay inside the
    // matrix and those rows only feed outputs that are never stored.
    const uint16_t *ap[ACH];
    const uint16_t *bp[BCH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        int64_t gm = m0 + r0 + i * ROWS_PER_PASS;
        gm = gm < M ? gm : M - 1;
        ap[i] = A + gm * lda + kc * 8;
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
        int64_t gn = n0 + r0 + i * ROWS_PER_PASS;
        gn = gn < N ? gn : N - 1;
        bp[i] = B + gn * ldb + kc * 8;
    }

    uint4 ra[ACH], rb[BCH];

    // Full K tile: plain 16-byte loads, no predicates.
    auto load_tiles_full = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            ra[i] = *(const uint4 *)(ap[i] + k0);
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            rb[i] = *(const uint4 *)(bp[i] + k0);
    };
    // Last, partial K tile: elements at k >= ke read as 0 (K-boundary mask).
    auto load_tiles_tail = [&](int64_t k0) {
        const int64_t gk = k0 + kc * 8;
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            ra[i] = load_chunk_tail(ap[i] - kc * 8, gk, ke);
#pragma unroll
        for (int i = 0; i < BCH; ++i)
            rb[i] = load_chunk_tail(bp[i] - kc * 8, gk, ke);
    };

    auto store_tiles = [&](int st) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int r = r0 + i * ROWS_PER_PASS;
            As[st * A_STAGE + r * 8 + (kc ^ ((r >> 1) & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int r = r0 + i * ROWS_PER_PASS;
            Bs[st * B_STAGE + r * 8 + (kc ^ ((r >> 1) & 7))] = rb[i];
        }
    };

    const int frag_row = lane & 31;       // row of A / column of B this lane feeds
    const int frag_half = lane >> 5;      // which 8 of the 16 k of one MFMA step
    const int swz = (frag_row >> 1) & 7;  // swizzle key of the fragment row (wave tiles are 32-aligned)

    // Fragments of one 16-deep k step: FM blocks of A, FN blocks of B.
    auto load_frags = [&](int st, int ks, bf16x8_t *af, bf16x8_t *bf) {
        const uint4 *as = As + st * A_STAGE + (wm * TM + frag_row) * 8;
        const uint4 *bs = Bs + st * B_STAGE + (wn * TN + frag_row) * 8;
        const int c = (ks * 2 + frag_half) ^ swz;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = __builtin_bit_cast(bf16x8_t, as[i * 32 * 8 + c]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = __builtin_bit_cast(bf16x8_t, bs[j * 32 * 8 + c]);
    };

    auto mfma_step = [&](const bf16x8_t *af, const bf16x8_t *bf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };

    // Fragment registers, two sets.  fa[1]/fb[1] carry the last k step of
    // the previous tile into the next iteration: its 16 MFMAs run after the
    // barrier, while the first fragment reads of the new tile are in flight.
    bf16x8_t fa[2][FM], fb[2][FN];

    // One LDS stage: the deferred step of the previous tile, then k steps
    // 0..2 of this tile, each while the next step's fragments are read;
    // step 3's fragments are left in fa[1]/fb[1].
    auto tile_body = [&](int st) {
        load_frags(st, 0, fa[0], fb[0]);
        mfma_step(fa[1], fb[1]);
        load_frags(st, 1, fa[1], fb[1]);
        mfma_step(fa[0], fb[0]);
        load_frags(st, 2, fa[0], fb[0]);
        mfma_step(fa[1], fb[1]);
        load_frags(st, 3, fa[1], fb[1]);
        mfma_step(fa[0], fb[0]);
    };

    // Instruction order of one steady-state iteration (after its global
    // loads): the first k step's fragment reads, then every MFMA paired with
    // one LDS read of the following step's fragments, and in the last
    // computed step every MFMA paired with one LDS write of the next tile,
    // so the matrix pipe does not wait on LDS traffic it could overlap.
    auto schedule_main_loop = [&]() {
        constexpr int kMfma = 0x008, kDsRead = 0x100, kDsWrite = 0x200;
        constexpr int kFrags = FM + FN, kMfmaPerStep = FM * FN;
        constexpr int kWrites = ACH + BCH;
        __builtin_amdgcn_sched_group_barrier(kDsRead, kFrags, 0);
#pragma unroll
        for (int step = 0; step < 3; ++step) {
#pragma unroll
            for (int i = 0; i < kMfmaPerStep; ++i) {
                __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
                if (i < kFrags)
                    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < kMfmaPerStep; ++i) {
            __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
            if (i < kWrites)
                __builtin_amdgcn_sched_group_barrier(kDsWrite, 1, 0);
        }
    };

    // K loop.  The steady-state loop runs while the next tile is a full
    // one; the last tile (partial when K is not a multiple of BK) is
    // loaded with the masked loader in the short loop after it, so the
    // steady state carries no predicates.
    const int64_t klen = ke > kb ? ke - kb : 0;
    const int64_t ntiles = (klen + MBK - 1) / MBK;
    const int64_t nfull = klen / MBK;
    if (g.alpha != 0.0f && ntiles > 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[1][i] = bf16x8_t{};
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[1][j] = bf16x8_t{};
        if (nfull > 0)
            load_tiles_full(kb);
        else
            load_tiles_tail(kb);
        store_tiles(0);
        __syncthreads();
        int64_t kt = 0;
        for (; kt + 1 < nfull; ++kt) {
            const int st = (int)(kt & 1);
            load_tiles_full(kb + (kt + 1) * MBK);
            // keep the next tile's global loads at the top of the iteration
            // so their latency overlaps this tile's MFMAs
            __builtin_amdgcn_sched_barrier(0);
            tile_body(st);
            store_tiles(st ^ 1);
            schedule_main_loop();
            __syncthreads();
        }
        for (; kt < ntiles; ++kt) {
            const int st = (int)(kt & 1);
            const bool has_next = kt + 1 < ntiles;   // then the next is the partial tile
            if (has_next)
                load_tiles_tail(kb + (kt + 1) * MBK);
            tile_body(st);
            if (has_next)
                store_tiles(st ^ 1);
            __syncthreads();
        }
        mfma_step(fa[1], fb[1]);   // last k step of the last tile
    }

    // Epilogue, in chunks of EP_ROWS tile rows: every wave writes the
    // accumulator blocks it owns in the chunk to LDS (the K loop's buffers
    // are free after its last barrier), then all threads store the chunk
    // along C's contiguous dimension.  In registers, lane l's value v of a
    // 32 x 32 block is row 8*(v/4) + 4*(l/32) + v%4, column l%32.
    constexpr int EP_ROWS = 64;
    constexpr int EP_LD = BN + 4;
    static_assert((EP_ROWS * EP_LD + BN) * 4 <= 2 * (BM + BN) * 8 * 16,
                  "epilogue chunk and bias fit in LDS");
    float *chunk = (float *)lds;
    // the tile's BN bias values, read from global memory once
    float *bias_s = chunk + EP_ROWS * EP_LD;
    if (g.bias && !g.write_partial) {
        for (int t = tid; t < BN; t += NT)
            bias_s[t] = n0 + t < N ? load_as_f32(g.bias, g.bias_bf16, n0 + t) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < BM / EP_ROWS; ++c) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row0 = wm * TM + i * 32 - c * EP_ROWS;   // block's first row in the chunk
            if (row0 >= 0 && row0 < EP_ROWS) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        chunk[(row0 + 8 * (v / 4) + 4 * frag_half + (v % 4)) * EP_LD + wn * TN +
                              j * 32 + (lane & 31)] = acc[i][j][v];
            }
        }
        __syncthreads();
        if (g.write_partial)
            store_chunk<4, true, false, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS,
                                                                  bias_s);
        else if (g.c_bf16)
            store_chunk<8, false, true, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS,
                                                                  bias_s);
        else
            store_chunk<4, false, false, EP_ROWS, BN, EP_LD, NT>(g, tc, chunk, m0, n0, c * EP_ROWS,
                                                                  bias_s);
        __syncthreads();
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_one(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const size_t lds_bytes = (size_t)2 * (BM + BN) * 8 * sizeof(uint4);
    auto kern = gemm_mfma_bf16_kernel<BM, BN, WM, WN>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.programs), dim3(64 * WM * WN), lds_bytes, stream,
                       g);
    return hipGetLastError();
}

} // namespace

// variant index -> instantiation
const TileConfig kMfmaBf16Tiles[] = {
    {256, 256, MBK, 256, 0, "mfma_bf16_256x256x64_w2x2"},
    {128, 128, MBK, 256, 1, "mfma_bf16_128x128x64_w2x2"},
    {256, 128, MBK, 256, 2, "mfma_bf16_256x128x64_w2x2"},
};
const int kNumMfmaBf16Tiles = 3;

hipError_t launch_mfma_bf16(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 0: return launch_one<256, 256, 2, 2>(g, p, stream);
    case 1: return launch_one<128, 128, 2, 2>(g, p, stream);
    case 2: return launch_one<256, 128, 2, 2>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
