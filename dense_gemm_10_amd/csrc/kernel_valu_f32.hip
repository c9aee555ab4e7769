// fp32 SGEMM on the vector ALUs: register-tiled outer product.
//
// Design ("La GEMM, de zero a cuBLAS" sections 2.4 - 2.8, rebuilt for
// wave64 CDNA4):
//   - block tile BM x BN = 128 x 128, BK = 16, 256 threads (4 wavefronts);
//   - each thread accumulates an 8 x 8 block of C in registers: per k it
//     reads 8 values of A and 8 of B from LDS and does 64 FMAs (the outer
//     product of section 2.6, 16 LDS words per 64 FMAs);
//   - A is staged in LDS transposed, As[k][m], so that both operands are
//     read as 128-bit vectors along m and n (section 2.7); the thread's 8
//     rows are two runs of 4 (ty*4 and 64 + ty*4) so a wavefront reads 4
//     distinct A vectors (broadcast) and 16 consecutive B vectors;
//   - global loads are 128-bit along each operand's contiguous dimension
//     (sections 2.3 and 2.7) and double-buffered: tile t+1 is fetched into
//     registers while tile t is multiplied out of LDS, then written to the
//     other LDS buffer, one barrier per K tile (section 2.8);
//   - loads are masked on the row/column bound and on the split's K range
//     with zero fill; stores are masked on M and N ("Skill: Write a Triton
//     GEMM Kernel", Required reasoning process step 5).
// The library is built without packed-fp32 instructions; the inner loop's
// FMAs are the two-operand accumulate form v_fmac_f32, which gfx950 issues
// at twice the rate of v_fma_f32: the ceiling is 128 FMA per clock per CU,
// the chip's published fp32 vector rate.
//
// Requirements checked on the host: fp32 A and B, 16-byte aligned base
// pointers, lda, ldb and batch strides multiples of 4 elements.
#include "launch.hpp"

namespace dg {

namespace {

constexpr int VBM = 128, VBN = 128, VBK = 16, VPAD = 4, VTHREADS = 256;

// Load 4 consecutive fp32 at p[off .. off+3]; element j exists iff
// line_ok && first + j < limit.  Missing elements read as 0.
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

template <bool A_COL, bool B_COL>
__global__ __launch_bounds__(VTHREADS, 2) void sgemm_valu_kernel(GemmArgs g)
{
    __shared__ __align__(16) float As[2][VBK][VBM + VPAD];
    __shared__ __align__(16) float Bs[2][VBK][VBN + VPAD];

    const TileCoord tc = decode_program(blockIdx.x, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * VBM;
    const int64_t n0 = (int64_t)tc.pid_n * VBN;
    int64_t kb, ke;
    split_range(g, tc.s, kb, ke);

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const float *A = (const float *)g.A + tc.b * g.sa;
    const float *B = (const float *)g.B + tc.b * g.sb;
    const int64_t M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.0f;

    float4 ra[2], rb[2];

    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (!A_COL) {      // A[m][k] at m*lda + k: 4 k per vector
                const int r = tid / 4 + 64 * e, kq = tid % 4;
                const int64_t gm = m0 + r, gk = k0 + kq * 4;
                ra[e] = load4_masked(A, gm * lda + gk, gm < M, gk, ke);
            } else {           // A[m][k] at k*lda + m: 4 m per vector
                const int k = tid / 32 + 8 * e, mq = tid % 32;
                const int64_t gk = k0 + k, gm = m0 + mq * 4;
                ra[e] = load4_masked(A, gk * lda + gm, gk < ke, gm, M);
            }
            if (!B_COL) {      // B[k][n] at k*ldb + n: 4 n per vector
                const int k = tid / 32 + 8 * e, nq = tid % 32;
                const int64_t gk = k0 + k, gn = n0 + nq * 4;
                rb[e] = load4_masked(B, gk * ldb + gn, gk < ke, gn, N);
            } else {           // B[k][n] at n*ldb + k: 4 k per vector
                const int n = tid / 4 + 64 * e, kq = tid % 4;
                const int64_t gn = n0 + n, gk = k0 + kq * 4;
                rb[e] = load4_masked(B, gn * ldb + gk, gn < N, gk, ke);
            }
        }
    };

    auto store_tiles = [&](int st) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (!A_COL) {
                const int r = tid / 4 + 64 * e, kq = tid % 4;
                As[st][kq * 4 + 0][r] = ra[e].x;
                As[st][kq * 4 + 1][r] = ra[e].y;
                As[st][kq * 4 + 2][r] = ra[e].z;
                As[st][kq * 4 + 3][r] = ra[e].w;
            } else {
                const int k = tid / 32 + 8 * e, mq = tid % 32;
                *(float4 *)&As[st][k][mq * 4] = ra[e];
            }
            if (!B_COL) {
                const int k = tid / 32 + 8 * e, nq = tid % 32;
                *(float4 *)&Bs[st][k][nq * 4] = rb[e];
            } else {
                const int n = tid / 4 + 64 * e, kq = tid % 4;
                Bs[st][kq * 4 + 0][n] = rb[e].x;
                Bs[st][kq * 4 + 1][n] = rb[e].y;
                Bs[st][kq * 4 + 2][n] = rb[e].z;
                Bs[st][kq * 4 + 3][n] = rb[e].w;
            }
        }
    };

    const int64_t nk = (ke > kb) ? (ke - kb + VBK - 1) / VBK : 0;
    if (g.alpha != 0.0f && nk > 0) {
        load_tiles(kb);
        store_tiles(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int st = (int)(kt & 1);
            if (kt + 1 < nk)
                load_tiles(kb + (kt + 1) * VBK);
            // Unrolled by 8, not 16: a full unroll lets the scheduler hoist
            // every LDS read of the tile and spill.
#pragma unroll 8
            for (int k = 0; k < VBK; ++k) {
                const float4 a0 = *(const float4 *)&As[st][k][ty * 4];
                const float4 a1 = *(const float4 *)&As[st][k][64 + ty * 4];
                const float4 b0 = *(const float4 *)&Bs[st][k][tx * 4];
                const float4 b1 = *(const float4 *)&Bs[st][k][64 + tx * 4];
                const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            if (kt + 1 < nk)
                store_tiles(st ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t gm = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
        if (gm >= M)
            continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t gn = n0 + (j < 4 ? tx * 4 + j : 64 + tx * 4 + (j - 4));
            if (gn < N)
                write_result(g, tc.b, tc.s, gm, gn, acc[i][j]);
        }
    }
}

} // namespace

const TileConfig kValuTiles[] = {
    {VBM, VBN, VBK, VTHREADS, 0, "valu_f32_128x128x16_t8x8"},
};
const int kNumValuTiles = 1;

hipError_t launch_valu_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.programs), block(VTHREADS);
    if (!g.a_col && !g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<false, false>), grid, block, 0, stream, g);
    else if (!g.a_col && g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<false, true>), grid, block, 0, stream, g);
    else if (g.a_col && !g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<true, false>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((sgemm_valu_kernel<true, true>), grid, block, 0, stream, g);
    return hipGetLastError();
}

} // namespace dg
