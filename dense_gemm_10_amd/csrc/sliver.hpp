// Columns past the last full tile of a wide output ("sliver" columns):
// the device code shared by the stand-alone sliver kernel
// (kernel_sliver.hip) and the 16-bit matrix-core kernel, which runs the
// one-column case as extra workgroups after its tiles.
//
// When N exceeds a multiple of the tile width by a few columns, the tiled
// kernels would spend a whole tile column (a full K loop per tile) on them
// and leave the last wave of tiles nearly empty.  The planner then runs the
// tiled kernel on the full tile columns and this code on the remaining
// nrem <= kMaxSliver columns.  Each output is a dot product of a row of A
// with a column of B ("La GEMM, de zero a cuBLAS", section 2.1: one output
// element per K-length product).  A wavefront takes kSliverRows rows of A:
// its 64 lanes stride along K in 16-byte pieces, and the loads of four K
// steps (the sliver columns' B pieces once, and every row's A piece) are
// issued before their FMAs, so a wavefront waits for memory once per four
// steps; every lane keeps rows x columns fp32 partial sums, the wavefront
// adds them up across lanes, and one lane per output applies the epilogue
// (alpha, beta * C, bias, activation, output dtype).
//
// Requirements checked on the host: row-major A with 16-byte aligned rows
// (lda a multiple of 16 bytes, aligned base).
#pragma once
#include "launch.hpp"

namespace dg {

template <int AB_TYPE>
__device__ __forceinline__ float elem_f32(const char *p, int64_t i)
{
    if (AB_TYPE == DT_F32)
        return ((const float *)p)[i];
    return half_to_f32<AB_TYPE>(((const uint16_t *)p)[i]);
}

// The VK values of a 16-byte piece as fp32.
template <int AB_TYPE, int VK>
__device__ __forceinline__ void unpack16(const uint4 q, float (&x)[VK])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < VK; ++e)
        x[e] = AB_TYPE == DT_F32 ? __uint_as_float(w[e])
                                 : half_to_f32<AB_TYPE>((uint16_t)(w[e / 2] >> (16 * (e % 2))));
}

// The 16-byte piece of row `p` (typed elements) at element k: one vector
// load when k + VK <= kend, else element by element with zero fill past
// kend.  `stride` is the distance between consecutive k (1, or the leading
// dimension of a row-major B column).
template <int AB_TYPE, int VK>
__device__ __forceinline__ uint4 piece16(const char *p, int64_t k, int64_t stride, int64_t kend,
                                         bool vec)
{
    if (vec && k + VK <= kend)
        return *(const uint4 *)(p + k * (16 / VK));
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < VK; ++e) {
        if (k + e < kend) {
            const int64_t i = (k + e) * stride;
            if (AB_TYPE == DT_F32)
                w[e] = ((const uint32_t *)p)[i];
            else
                w[e / 2] |= (uint32_t)((const uint16_t *)p)[i] << (16 * (e % 2));
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rows [blk * kSliverRowsPerBlock, + kSliverRowsPerBlock) of batch entry b,
// columns [n0, n0 + nrem) (nrem <= NR), by the workgroup's 256 threads.
// Uses no LDS and no barrier.
template <int AB_TYPE, int NR>
__device__ __forceinline__ void sliver_block(const GemmArgs &g, int64_t n0, int32_t nrem, int64_t blk,
                                             int64_t b)
{
    constexpr int ES = AB_TYPE == DT_F32 ? 4 : 2;   // element size
    constexpr int VK = 16 / ES;                     // K elements per 16-byte piece
    constexpr int R = kSliverRows;
    static_assert(R * NR <= 64, "one lane per output");
    const int lane = threadIdx.x & 63;
    const int64_t m0 = (blk * (kSliverThreads / 64) + (threadIdx.x >> 6)) * R;
    if (m0 >= g.M)
        return;                                     // whole wavefronts leave together
    const char *A = (const char *)g.A + b * g.sa * ES;
    const char *B = (const char *)g.B + b * g.sb * ES;
    // B's sliver columns K-contiguous with 16-byte aligned starts
    const bool b_vec = g.b_col && ((((uintptr_t)B + (uintptr_t)(n0 * g.ldb * ES)) |
                                    (uintptr_t)(g.ldb * ES)) & 15) == 0;
    float acc[R][NR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NR; ++j)
            acc[r][j] = 0.0f;
    // kSteps K steps at a time, every load of them issued before the first
    // FMA (kept as raw 16-byte pieces until then), so a wavefront waits for
    // memory once per kSteps steps: for K up to 2048 16-bit elements, once
    constexpr int kSteps = 4;
    for (int64_t kc = (int64_t)lane * VK; kc < g.K; kc += kSteps * 64 * VK) {
        uint4 bq[kSteps][NR], aq[kSteps][R];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const int64_t k = kc + (int64_t)st * 64 * VK;
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                const int64_t n = n0 + (j < nrem ? j : 0);
                // column n of B: K-contiguous (b_col) or one element per row
                const char *col = g.b_col ? B + n * g.ldb * ES : B + n * ES;
                bq[st][j] = j < nrem ? piece16<AB_TYPE, VK>(col, k, g.b_col ? 1 : g.ldb, g.K, b_vec)
                                     : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t m = m0 + r < g.M ? m0 + r : g.M - 1;   // rows past M: any valid row, unused
                aq[st][r] = piece16<AB_TYPE, VK>(A + m * g.lda * ES, k, 1, g.K, true);
            }
        }
        // in K order: step by step, element by element
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            float bv[NR][VK];
#pragma unroll
            for (int j = 0; j < NR; ++j)
                unpack16<AB_TYPE, VK>(bq[st][j], bv[j]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float av[VK];
                unpack16<AB_TYPE, VK>(aq[st][r], av);
#pragma unroll
                for (int j = 0; j < NR; ++j)
#pragma unroll
                    for (int e = 0; e < VK; ++e)
                        acc[r][j] = fmaf(av[e], bv[j][e], acc[r][j]);
            }
        }
    }
    // sum over the wavefront's 64 lanes
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NR; ++j) {
            if (j >= nrem)
                break;
            float v = acc[r][j];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                v += __shfl_xor(v, off, 64);
            acc[r][j] = v;
        }
    // lane r * NR + j finishes output (m0 + r, n0 + j)
    const int r = lane / NR, j = lane % NR;
    if (lane < R * NR && j < nrem && m0 + r < g.M) {
        float v = 0.0f;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
            for (int jj = 0; jj < NR; ++jj)
                if (rr == r && jj == j)
                    v = acc[rr][jj];
        const int64_t m = m0 + r, n = n0 + j;
        store_c(g, b, m, n, epilogue_value(g, b, m, n, v));
    }
}

} // namespace dg
