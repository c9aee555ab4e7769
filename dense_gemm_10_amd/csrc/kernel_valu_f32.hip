// fp32 SGEMM on the vector ALUs: register-tiled outer product.
//
// Design ("La GEMM, de zero a cuBLAS" sections 2.4 - 2.8, rebuilt for
// wave64 CDNA4):
//   - 256 threads (4 wavefronts) as a 16 x 16 grid; each thread
//     accumulates an 8 x TN block of C in registers, so the block tile is
//     BM x BN = 128 x 16 TN (TN = 8: 128 x 128, TN = 16: 128 x 256), with
//     BK = 16;
//   - per k a thread reads 8 values of A and TN of B from LDS and does 8 TN
//     FMAs (the outer product of section 2.6): 16 LDS words per 64 FMAs at
//     TN = 8, 24 per 128 at TN = 16.  At two wavefronts per SIMD the
//     8 x 8 tile's LDS reads take about as long as its FMAs; the 8 x 16
//     tile cuts them by a quarter per FMA;
//   - A is staged in LDS transposed, As[k][m], so that both operands are
//     read as 128-bit vectors along m and n (section 2.7); a thread's rows
//     are two runs of 4 (ty*4 and 64 + ty*4) and its columns TN / 4 runs of
//     4 (tx*4 + 64 j), so a wavefront reads 4 distinct A vectors
//     (broadcast) and 16 consecutive B vectors per run;
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

constexpr int VBM = 128, VBK = 16, VPAD = 4, VTHREADS = 256;

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

// Operand tile of R x VBK (R = rows of the operand along M or N) in
// float4 vectors: along the K-contiguous dimension a vector holds 4 k of
// one row, otherwise 4 rows of one k.  Vector e (0 <= e < R / 64) of
// thread tid covers row / k coordinates returned by these helpers.
template <int R>
struct VTile {
    static constexpr int kVecs = R / 64;                 // vectors per thread
    // K-contiguous: row tid / 4 + 64 e, k 4 (tid % 4) .. + 3
    __device__ static int kc_row(int tid, int e) { return tid / 4 + 64 * e; }
    __device__ static int kc_k(int tid) { return (tid % 4) * 4; }
    // R-contiguous: k tid / (R / 4) + (1024 / R) e, rows 4 (tid % (R / 4)) .. + 3
    __device__ static int rc_k(int tid, int e) { return tid / (R / 4) + (1024 / R) * e; }
    __device__ static int rc_row(int tid) { return (tid % (R / 4)) * 4; }
};

template <int TN, bool A_COL, bool B_COL>
__global__ __launch_bounds__(VTHREADS, 2) void sgemm_valu_kernel(GemmArgs g)
{
    constexpr int VBN = 16 * TN;
    constexpr int NA = VTile<VBM>::kVecs, NB = VTile<VBN>::kVecs;
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

    float acc[8][TN];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = 0.0f;

    float4 ra[NA], rb[NB];

    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            if (!A_COL) {      // A[m][k] at m*lda + k: 4 k per vector
                const int64_t gm = m0 + VTile<VBM>::kc_row(tid, e), gk = k0 + VTile<VBM>::kc_k(tid);
                ra[e] = load4_masked(A, gm * lda + gk, gm < M, gk, ke);
            } else {           // A[m][k] at k*lda + m: 4 m per vector
                const int64_t gk = k0 + VTile<VBM>::rc_k(tid, e), gm = m0 + VTile<VBM>::rc_row(tid);
                ra[e] = load4_masked(A, gk * lda + gm, gk < ke, gm, M);
            }
        }
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            if (!B_COL) {      // B[k][n] at k*ldb + n: 4 n per vector
                const int64_t gk = k0 + VTile<VBN>::rc_k(tid, e), gn = n0 + VTile<VBN>::rc_row(tid);
                rb[e] = load4_masked(B, gk * ldb + gn, gk < ke, gn, N);
            } else {           // B[k][n] at n*ldb + k: 4 k per vector
                const int64_t gn = n0 + VTile<VBN>::kc_row(tid, e), gk = k0 + VTile<VBN>::kc_k(tid);
                rb[e] = load4_masked(B, gn * ldb + gk, gn < N, gk, ke);
            }
        }
    };

    auto store_tiles = [&](int st) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            if (!A_COL) {
                const int r = VTile<VBM>::kc_row(tid, e), k = VTile<VBM>::kc_k(tid);
                As[st][k + 0][r] = ra[e].x;
                As[st][k + 1][r] = ra[e].y;
                As[st][k + 2][r] = ra[e].z;
                As[st][k + 3][r] = ra[e].w;
            } else {
                *(float4 *)&As[st][VTile<VBM>::rc_k(tid, e)][VTile<VBM>::rc_row(tid)] = ra[e];
            }
        }
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            if (!B_COL) {
                *(float4 *)&Bs[st][VTile<VBN>::rc_k(tid, e)][VTile<VBN>::rc_row(tid)] = rb[e];
            } else {
                const int n = VTile<VBN>::kc_row(tid, e), k = VTile<VBN>::kc_k(tid);
                Bs[st][k + 0][n] = rb[e].x;
                Bs[st][k + 1][n] = rb[e].y;
                Bs[st][k + 2][n] = rb[e].z;
                Bs[st][k + 3][n] = rb[e].w;
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
                const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                float b[TN];
#pragma unroll
                for (int j = 0; j < TN / 4; ++j) {
                    const float4 bj = *(const float4 *)&Bs[st][k][64 * j + tx * 4];
                    b[4 * j] = bj.x; b[4 * j + 1] = bj.y; b[4 * j + 2] = bj.z; b[4 * j + 3] = bj.w;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
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
        for (int j = 0; j < TN; ++j) {
            const int64_t gn = n0 + 64 * (j / 4) + tx * 4 + (j % 4);
            if (gn < N)
                write_result(g, tc.b, tc.s, gm, gn, acc[i][j]);
        }
    }
}

template <int TN>
void launch_valu_tn(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.programs), block(VTHREADS);
    if (!g.a_col && !g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<TN, false, false>), grid, block, 0, stream, g);
    else if (!g.a_col && g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<TN, false, true>), grid, block, 0, stream, g);
    else if (g.a_col && !g.b_col)
        hipLaunchKernelGGL((sgemm_valu_kernel<TN, true, false>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((sgemm_valu_kernel<TN, true, true>), grid, block, 0, stream, g);
}

} // namespace

// variant = TN (columns per thread)
const TileConfig kValuTiles[] = {
    {VBM, 128, VBK, VTHREADS, 8, "valu_f32_128x128x16_t8x8"},
    {VBM, 256, VBK, VTHREADS, 16, "valu_f32_128x256x16_t8x16"},
};
const int kNumValuTiles = 2;

hipError_t launch_valu_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    if (p.tile.variant == 16)
        launch_valu_tn<16>(g, p, stream);
    else
        launch_valu_tn<8>(g, p, stream);
    return hipGetLastError();
}

} // namespace dg
