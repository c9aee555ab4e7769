// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32): fp32 inputs,
// fp32 products and accumulation.
//
// Same tiling as the other kernels ("La GEMM, de zero a cuBLAS", the three
// tiling levels of section 2.6: workgroup tile in LDS, wave tile in
// registers, 32 x 32 MFMA blocks), for every operand order:
//   - tile BM x BN, BK = 16 or 32, 4 wavefronts in a 2 x 2 layout; each wave owns
//     a (BM/2) x (BN/2) tile of 32 x 32 blocks in fp32 accumulators;
//   - A is staged in LDS as As[k][m] and B as Bs[k][n] (section 2.7's
//     transposed A), so the operand an MFMA lane needs - row (l mod 32) of
//     A and column (l mod 32) of B at k = 2s + l/32 - is one float read by
//     32 consecutive lanes from consecutive addresses;
//   - global loads are 128-bit along each operand's contiguous dimension,
//     masked on the row / column bound and the split's K range only in
//     edge tiles, and double-buffered through registers: tile t+1 is
//     fetched while tile t is multiplied and written to the other LDS stage
//     half-way through it, one barrier per K tile (section 2.8);
//   - inside a K tile the fragment reads of each k-step are interleaved
//     with the MFMAs of the previous one.
// A 32x32x2 fp32 MFMA does 4096 flops in 64 cycles; per BK-deep K tile a
// wave issues BK/2 k-steps of FM*FN MFMAs against BK/2*(FM+FN) one-float
// LDS reads, so the kernel is bound by the matrix pipe, not by memory.  A
// 32-deep K tile halves the barriers and stage hand-offs per K.
//
// Requirements checked on the host: fp32 A and B, 16-byte aligned base
// pointers, lda, ldb and batch strides multiples of 4 elements.
#include "epilogue.hpp"
#include "launch.hpp"

namespace dg {

namespace {

constexpr int FPAD = 4;

// 4 consecutive fp32 at p[off .. off+3]; element j exists iff line_ok &&
// first + j < limit.  Missing elements read as 0.
__device__ __forceinline__ float4 load4_masked(const float *p, int64_t off, bool line_ok,
                                               int64_t first, int64_t limit)
{
    if (line_ok && first + 3 < limit)
        return *(const float4 *)(p + off);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (line_ok) {
        if (first + 0 < limit) v.x = p[off + 0];
        if (first + 1 < limit) v.y = p[off + 1];
        if (first + 2 < limit) v.z = p[off + 2];
        if (first + 3 < limit) v.w = p[off + 3];
    }
    return v;
}

template <int BM, int BN, int WM, int WN, int FBK, bool A_COL, bool B_COL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_f32_kernel(GemmArgs g)
{
    constexpr int KQ = FBK / 4;                            // 128-bit vectors per K-contiguous line
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int KSTEPS = FBK / 2;                        // MFMA k-steps per K tile
    constexpr int ALD = BM + FPAD, BLD = BN + FPAD;       // LDS row strides (floats)
    constexpr int A_STAGE = FBK * ALD, B_STAGE = FBK * BLD;
    // 128-bit loads per thread per K tile
    constexpr int A_VEC = BM * FBK / 4 / NT, B_VEC = BN * FBK / 4 / NT;
    static_assert(A_VEC * NT * 4 == BM * FBK && B_VEC * NT * 4 == BN * FBK, "load split");
    static_assert(FM + FN <= FM * FN, "fragment reads fit in the slots");

    extern __shared__ float smem[];
    float *As = smem;                    // [2][FBK][ALD]
    float *Bs = smem + 2 * A_STAGE;      // [2][FBK][BLD]

    const TileCoord tc = decode_program(blockIdx.x, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * BM;
    const int64_t n0 = (int64_t)tc.pid_n * BN;
    int64_t kb, ke;
    split_range(g, tc.s, kb, ke);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const float *A = (const float *)g.A + tc.b * g.sa;
    const float *B = (const float *)g.B + tc.b * g.sb;
    const int64_t M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;
    // every row and column of the tile inside the matrices: no M / N masks
    const bool interior = m0 + BM <= M && n0 + BN <= N;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x16_t{};

    float4 ra[A_VEC], rb[B_VEC];

    // Global -> registers, vector e (A vectors first, then B) of the K tile
    // at k0, when the whole tile, K range included, lies inside the
    // operands.  Issued one at a time between MFMAs (see tile_body).
    constexpr int NVEC = A_VEC + B_VEC;
    auto load_one = [&](int e, int64_t k0) {
        if (e < A_VEC) {
            const int idx = tid + e * NT;
            if (!A_COL) {
                const int r = idx / KQ, kq = idx % KQ;
                ra[e] = *(const float4 *)(A + (m0 + r) * lda + k0 + kq * 4);
            } else {
                const int k = idx / (BM / 4), mq = idx % (BM / 4);
                ra[e] = *(const float4 *)(A + (k0 + k) * lda + m0 + mq * 4);
            }
        } else {
            const int idx = tid + (e - A_VEC) * NT;
            if (!B_COL) {
                const int k = idx / (BN / 4), nq = idx % (BN / 4);
                rb[e - A_VEC] = *(const float4 *)(B + (k0 + k) * ldb + n0 + nq * 4);
            } else {
                const int n = idx / KQ, kq = idx % KQ;
                rb[e - A_VEC] = *(const float4 *)(B + (n0 + n) * ldb + k0 + kq * 4);
            }
        }
    };
    // The whole K tile at k0 with the row / column and K masks (edge tiles).
    auto load_tiles_masked = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < A_VEC; ++e) {
            const int idx = tid + e * NT;
            if (!A_COL) {            // A[m][k] at m*lda + k: 4 k per vector
                const int r = idx / KQ, kq = idx % KQ;
                const int64_t gm = m0 + r, gk = k0 + kq * 4;
                ra[e] = load4_masked(A, gm * lda + gk, gm < M, gk, ke);
            } else {                 // A[m][k] at k*lda + m: 4 m per vector
                const int k = idx / (BM / 4), mq = idx % (BM / 4);
                const int64_t gk = k0 + k, gm = m0 + mq * 4;
                ra[e] = load4_masked(A, gk * lda + gm, gk < ke, gm, M);
            }
        }
#pragma unroll
        for (int e = 0; e < B_VEC; ++e) {
            const int idx = tid + e * NT;
            if (!B_COL) {            // B[k][n] at k*ldb + n: 4 n per vector
                const int k = idx / (BN / 4), nq = idx % (BN / 4);
                const int64_t gk = k0 + k, gn = n0 + nq * 4;
                rb[e] = load4_masked(B, gk * ldb + gn, gk < ke, gn, N);
            } else {                 // B[k][n] at n*ldb + k: 4 k per vector
                const int n = idx / KQ, kq = idx % KQ;
                const int64_t gn = n0 + n, gk = k0 + kq * 4;
                rb[e] = load4_masked(B, gn * ldb + gk, gn < N, gk, ke);
            }
        }
    };

    // Registers -> LDS stage st, vector e (A vectors first, then B).
    auto store_one = [&](int st, int e) {
        float *as = As + st * A_STAGE;
        float *bs = Bs + st * B_STAGE;
        if (e < A_VEC) {
            const int idx = tid + e * NT;
            if (!A_COL) {
                const int r = idx / KQ, kq = idx % KQ;
                as[(kq * 4 + 0) * ALD + r] = ra[e].x;
                as[(kq * 4 + 1) * ALD + r] = ra[e].y;
                as[(kq * 4 + 2) * ALD + r] = ra[e].z;
                as[(kq * 4 + 3) * ALD + r] = ra[e].w;
            } else {
                const int k = idx / (BM / 4), mq = idx % (BM / 4);
                *(float4 *)&as[k * ALD + mq * 4] = ra[e];
            }
        } else {
            const int idx = tid + (e - A_VEC) * NT;
            const float4 v = rb[e - A_VEC];
            if (!B_COL) {
                const int k = idx / (BN / 4), nq = idx % (BN / 4);
                *(float4 *)&bs[k * BLD + nq * 4] = v;
            } else {
                const int n = idx / KQ, kq = idx % KQ;
                bs[(kq * 4 + 0) * BLD + n] = v.x;
                bs[(kq * 4 + 1) * BLD + n] = v.y;
                bs[(kq * 4 + 2) * BLD + n] = v.z;
                bs[(kq * 4 + 3) * BLD + n] = v.w;
            }
        }
    };
    auto store_tiles = [&](int st) {
#pragma unroll
        for (int e = 0; e < NVEC; ++e)
            store_one(st, e);
    };

    // Fragments alternate between two register sets per k-step; fa[1] /
    // fb[1] carry the last k-step of a tile across the barrier, where its
    // MFMAs run while the next tile's first fragments are read.
    const int frag = lane & 31, khalf = lane >> 5;
    float fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
        fa[1][i] = 0.0f;
#pragma unroll
    for (int j = 0; j < FN; ++j)
        fb[1][j] = 0.0f;

    // One K tile from stage st, as KSTEPS k-steps of FM * FN fenced slots:
    // slot n issues the MFMA of block n on the previous k-step's fragments
    // and, in the first FM + FN slots, the read of one fragment of this
    // k-step (left alone, the compiler sinks the reads next to their use and
    // the LDS latency stalls the matrix pipe).  When the next tile is
    // loaded without masks (load_next), its global loads are issued one
    // every SPREAD slots from the start of the tile, and its LDS stores one
    // every SPREAD slots from k-step STORE_STEP: issued as one block, the
    // loads of the four waves kept the matrix pipe idle for about a fifth
    // of the loop.  Edge tiles load the next tile as one masked block
    // before the body and store it at STORE_STEP (store_next).
    constexpr int SLOTS = KSTEPS * FM * FN;
    constexpr int SPREAD = 2;
    constexpr int STORE_STEP = KSTEPS / 2;
    static_assert(NVEC * SPREAD <= STORE_STEP * FM * FN, "loads issued before the stores");
    static_assert(STORE_STEP * FM * FN + NVEC * SPREAD <= SLOTS, "stores inside the tile");
    auto tile_body = [&](int st, bool load_next, int64_t k_next, bool store_next) {
        const float *as = As + st * A_STAGE + wm * TM + frag;
        const float *bs = Bs + st * B_STAGE + wn * TN + frag;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const int cur = s & 1, prev = cur ^ 1;
            const int k = 2 * s + khalf;
#pragma unroll
            for (int n = 0; n < FM * FN; ++n) {
                if (n < FM)
                    fa[cur][n] = as[k * ALD + n * 32];
                else if (n < FM + FN)
                    fb[cur][n - FM] = bs[k * BLD + (n - FM) * 32];
                const int i = n / FN, j = n % FN;
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[prev][i], fb[prev][j],
                                                                 acc[i][j], 0, 0, 0);
                const int slot = s * FM * FN + n;
                if (load_next && slot % SPREAD == SPREAD - 1 && slot / SPREAD < NVEC)
                    load_one(slot / SPREAD, k_next);
                const int ss = slot - STORE_STEP * FM * FN;
                if ((load_next || store_next) && ss >= 0 && ss % SPREAD == SPREAD - 1 &&
                    ss / SPREAD < NVEC)
                    store_one(st ^ 1, ss / SPREAD);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    const int64_t nk = (ke > kb) ? (ke - kb + FBK - 1) / FBK : 0;
    const int64_t nk_full = (ke - kb) / FBK;   // K tiles with all FBK k inside the split
    if (g.alpha != 0.0f && nk > 0) {
        if (interior && nk_full >= 1) {
#pragma unroll
            for (int e = 0; e < NVEC; ++e)
                load_one(e, kb);
        } else {
            load_tiles_masked(kb);
        }
        store_tiles(0);
        int64_t kt = 0;
        // Steady state of an interior tile: the next K tile is whole, its
        // loads are unmasked and spread over this tile's body.  With the
        // flags constant the body has no branches, and the compiler counts
        // outstanding loads exactly; behind runtime flags it waited for all
        // of them (vmcnt(0)) in the middle of the matrix work.
        if (interior) {
            for (; kt + 1 < nk_full; ++kt) {
                lds_barrier();
                tile_body((int)(kt & 1), true, kb + (kt + 1) * FBK, false);
            }
        }
        for (; kt < nk; ++kt) {
            const int st = (int)(kt & 1);
            const bool has_next = kt + 1 < nk;
            const bool fast_next = has_next && interior && kt + 1 < nk_full;
            const int64_t k_next = kb + (kt + 1) * FBK;
            lds_barrier();   // stage st complete; the stage written next no longer read
            if (has_next && !fast_next)
                load_tiles_masked(k_next);
            tile_body(st, fast_next, k_next, has_next && !fast_next);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)   // last k-step of the last tile
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1][i], fb[1][j], acc[i][j],
                                                                 0, 0, 0);
        lds_barrier();
    }

    // the launch gives the kernel max(loop buffers, epilogue) bytes of LDS
    // 256 x 256 tiles run one workgroup per CU (512 registers per lane),
    // 128 x 128 tiles two
    tile_epilogue<BM, BN, WM, WN, (BM * BN >= 256 * 256 ? 512 : 256)>(g, tc, smem, m0, n0, acc);
}

template <int BM, int BN, int WM, int WN, int FBK>
size_t f32_lds_bytes()
{
    const size_t loop = (size_t)2 * FBK * ((BM + FPAD) + (BN + FPAD)) * sizeof(float);
    const size_t epi = (size_t)epilogue_lds_bytes(BN);
    return loop > epi ? loop : epi;
}

template <int BM, int BN, int WM, int WN, int FBK>
hipError_t launch_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const size_t lds = f32_lds_bytes<BM, BN, WM, WN, FBK>();
    dim3 grid((unsigned)p.programs), block(64 * WM * WN);
    if (!g.a_col && !g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, FBK, false, false>), grid, block, lds,
                           stream, g);
    else if (!g.a_col && g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, FBK, false, true>), grid, block, lds,
                           stream, g);
    else if (g.a_col && !g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, FBK, true, false>), grid, block, lds,
                           stream, g);
    else
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, FBK, true, true>), grid, block, lds,
                           stream, g);
    return hipGetLastError();
}

} // namespace

// Entries 0 and 1 are the large and small tiles of the automatic choice;
// the 32-deep ones are selectable by name and by the tuned table.
hipError_t launch_mfma_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 0: return launch_f32<256, 256, 2, 2, 16>(g, p, stream);
    case 1: return launch_f32<128, 128, 2, 2, 16>(g, p, stream);
    case 2: return launch_f32<256, 256, 2, 2, 32>(g, p, stream);
    case 3: return launch_f32<128, 128, 2, 2, 32>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
