// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32): fp32 inputs,
// fp32 products and accumulation.
//
// Same tiling as the other kernels ("La GEMM, de zero a cuBLAS", the three
// tiling levels of section 2.6: workgroup tile in LDS, wave tile in
// registers, 32 x 32 MFMA blocks), for every operand order:
//   - tile BM x BN, BK = 16, 4 wavefronts in a 2 x 2 layout; each wave owns
//     a (BM/2) x (BN/2) tile of 32 x 32 blocks in fp32 accumulators;
//   - A is staged in LDS as As[k][m] and B as Bs[k][n] (section 2.7's
//     transposed A), so the operand an MFMA lane needs - row (l mod 32) of
//     A and column (l mod 32) of B at k = 2s + l/32 - is one float read by
//     32 consecutive lanes from consecutive addresses;
//   - global loads are 128-bit along each operand's contiguous dimension,
//     masked on the row / column bound and the split's K range, and
//     double-buffered through registers: tile t+1 is fetched while tile t
//     is multiplied, one barrier per K tile (section 2.8).
// A 32x32x2 fp32 MFMA does 4096 flops in 64 cycles; per 16-deep K tile a
// wave issues 8 k-steps of FM*FN MFMAs against 8*(FM+FN) one-float LDS
// reads, so the kernel is bound by the matrix pipe, not by memory.
//
// Requirements checked on the host: fp32 A and B, 16-byte aligned base
// pointers, lda, ldb and batch strides multiples of 4 elements.
#include "epilogue.hpp"
#include "launch.hpp"

namespace dg {

namespace {

constexpr int FBK = 16;
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

template <int BM, int BN, int WM, int WN, bool A_COL, bool B_COL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_f32_kernel(GemmArgs g)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ALD = BM + FPAD, BLD = BN + FPAD;       // LDS row strides (floats)
    constexpr int A_STAGE = FBK * ALD, B_STAGE = FBK * BLD;
    // 128-bit loads per thread per K tile
    constexpr int A_VEC = BM * FBK / 4 / NT, B_VEC = BN * FBK / 4 / NT;
    static_assert(A_VEC * NT * 4 == BM * FBK && B_VEC * NT * 4 == BN * FBK, "load split");

    extern __shared__ float smem[];
    float *As = smem;                    // [2][FBK][ALD]
    float *Bs = smem + 2 * A_STAGE;      // [2][FBK][BLD]

    const TileCoord tc = decode_program(blockIdx.x, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * BM;
    const int64_t n0 = (int64_t)tc.pid_n * BN;
    int64_t kb, ke;
    split_range(g, tc.s, kb, ke);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const float *A = (const float *)g.A + tc.b * g.sa;
    const float *B = (const float *)g.B + tc.b * g.sb;
    const int64_t M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    float4 ra[A_VEC], rb[B_VEC];

    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < A_VEC; ++e) {
            const int idx = tid + e * NT;
            if (!A_COL) {            // A[m][k] at m*lda + k: 4 k per vector
                const int r = idx / 4, kq = idx % 4;
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
                const int n = idx / 4, kq = idx % 4;
                const int64_t gn = n0 + n, gk = k0 + kq * 4;
                rb[e] = load4_masked(B, gn * ldb + gk, gn < N, gk, ke);
            }
        }
    };

    auto store_tiles = [&](int st) {
        float *as = As + st * A_STAGE;
        float *bs = Bs + st * B_STAGE;
#pragma unroll
        for (int e = 0; e < A_VEC; ++e) {
            const int idx = tid + e * NT;
            if (!A_COL) {
                const int r = idx / 4, kq = idx % 4;
                as[(kq * 4 + 0) * ALD + r] = ra[e].x;
                as[(kq * 4 + 1) * ALD + r] = ra[e].y;
                as[(kq * 4 + 2) * ALD + r] = ra[e].z;
                as[(kq * 4 + 3) * ALD + r] = ra[e].w;
            } else {
                const int k = idx / (BM / 4), mq = idx % (BM / 4);
                *(float4 *)&as[k * ALD + mq * 4] = ra[e];
            }
        }
#pragma unroll
        for (int e = 0; e < B_VEC; ++e) {
            const int idx = tid + e * NT;
            if (!B_COL) {
                const int k = idx / (BN / 4), nq = idx % (BN / 4);
                *(float4 *)&bs[k * BLD + nq * 4] = rb[e];
            } else {
                const int n = idx / 4, kq = idx % 4;
                bs[(kq * 4 + 0) * BLD + n] = rb[e].x;
                bs[(kq * 4 + 1) * BLD + n] = rb[e].y;
                bs[(kq * 4 + 2) * BLD + n] = rb[e].z;
                bs[(kq * 4 + 3) * BLD + n] = rb[e].w;
            }
        }
    };

    const int frag = lane & 31, khalf = lane >> 5;
    auto compute = [&](int st) {
        const float *as = As + st * A_STAGE + wm * TM + frag;
        const float *bs = Bs + st * B_STAGE + wn * TN + frag;
#pragma unroll
        for (int s = 0; s < FBK / 2; ++s) {
            const int k = 2 * s + khalf;
            float a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = as[k * ALD + i * 32];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = bs[k * BLD + j * 32];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int64_t nk = (ke > kb) ? (ke - kb + FBK - 1) / FBK : 0;
    if (g.alpha != 0.0f && nk > 0) {
        load_tiles(kb);
        store_tiles(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int st = (int)(kt & 1);
            if (kt + 1 < nk)
                load_tiles(kb + (kt + 1) * FBK);
            compute(st);
            if (kt + 1 < nk)
                store_tiles(st ^ 1);
            __syncthreads();
        }
    }

    // the launch gives the kernel max(loop buffers, epilogue) bytes of LDS
    tile_epilogue<BM, BN, WM, WN>(g, tc, smem, m0, n0, acc);
}

template <int BM, int BN, int WM, int WN>
size_t f32_lds_bytes()
{
    const size_t loop = (size_t)2 * FBK * ((BM + FPAD) + (BN + FPAD)) * sizeof(float);
    const size_t epi = (size_t)epilogue_lds_bytes(BN);
    return loop > epi ? loop : epi;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const size_t lds = f32_lds_bytes<BM, BN, WM, WN>();
    dim3 grid((unsigned)p.programs), block(64 * WM * WN);
    if (!g.a_col && !g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, false, false>), grid, block, lds,
                           stream, g);
    else if (!g.a_col && g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, false, true>), grid, block, lds,
                           stream, g);
    else if (g.a_col && !g.b_col)
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, true, false>), grid, block, lds,
                           stream, g);
    else
        hipLaunchKernelGGL((gemm_mfma_f32_kernel<BM, BN, WM, WN, true, true>), grid, block, lds,
                           stream, g);
    return hipGetLastError();
}

} // namespace

const TileConfig kMfmaF32Tiles[] = {
    {256, 256, FBK, 256, 0, "mfma_f32_256x256x16_w2x2"},
    {128, 128, FBK, 256, 1, "mfma_f32_128x128x16_w2x2"},
};
const int kNumMfmaF32Tiles = 2;

hipError_t launch_mfma_f32(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    switch (p.tile.variant) {
    case 0: return launch_f32<256, 256, 2, 2>(g, p, stream);
    case 1: return launch_f32<128, 128, 2, 2>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
