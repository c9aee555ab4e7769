// Columns past the last full tile of a wide output ("sliver" columns).
//
// When N exceeds a multiple of the tile width by a few columns, the tiled
// kernels would spend a whole tile column (a full K loop per tile) on them
// and leave the last wave of tiles nearly empty.  The planner then runs the
// tiled kernel on the full tile columns and this kernel on the remaining
// nrem <= kMaxSliver columns.  Each output is a dot product of a row of A
// with a column of B ("La GEMM, de zero a cuBLAS", section 2.1: one output
// element per K-length product), so one wavefront takes one row m: its 64
// lanes stride along K with 16-byte loads of the K-contiguous A row, every
// lane keeps nrem fp32 partial sums, the wavefront adds them up across
// lanes, and the epilogue (alpha, beta * C, bias, activation, output
// dtype) is applied once per output.
//
// Requirements checked on the host: row-major A with 16-byte aligned rows
// (lda a multiple of 16 bytes, aligned base).
#include "launch.hpp"

namespace dg {

namespace {

constexpr int kSliverThreads = 256;        // 4 rows per workgroup

template <int AB_TYPE>
__device__ __forceinline__ float elem_f32(const void *p, int64_t i)
{
    if (AB_TYPE == DT_F32)
        return ((const float *)p)[i];
    return half_to_f32<AB_TYPE>(((const uint16_t *)p)[i]);
}

template <int AB_TYPE>
__global__ __launch_bounds__(kSliverThreads) void gemm_sliver_kernel(GemmArgs g, int64_t n0,
                                                                     int32_t nrem)
{
    constexpr int VK = AB_TYPE == DT_F32 ? 4 : 8;   // K elements per 16-byte load
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * (kSliverThreads / 64) + (threadIdx.x >> 6);
    const int64_t b = blockIdx.y;
    if (m >= g.M)
        return;                                     // whole wavefronts leave together
    const char *arow = (const char *)g.A +
                       (b * g.sa + m * g.lda) * (AB_TYPE == DT_F32 ? 4 : 2);
    const void *B = (const char *)g.B + b * g.sb * (AB_TYPE == DT_F32 ? 4 : 2);
    float acc[kMaxSliver];
#pragma unroll
    for (int j = 0; j < kMaxSliver; ++j)
        acc[j] = 0.0f;
    for (int64_t k = (int64_t)lane * VK; k < g.K; k += 64 * VK) {
        float a[VK];
        if (k + VK <= g.K) {
            const uint4 q = *(const uint4 *)(arow + k * (AB_TYPE == DT_F32 ? 4 : 2));
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < VK; ++e)
                a[e] = AB_TYPE == DT_F32 ? __uint_as_float(w[e])
                                         : half_to_f32<AB_TYPE>((uint16_t)(w[e / 2] >> (16 * (e % 2))));
        } else {
#pragma unroll
            for (int e = 0; e < VK; ++e)
                a[e] = k + e < g.K ? elem_f32<AB_TYPE>(arow, k + e) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kMaxSliver; ++j) {
            if (j >= nrem)
                break;
            const int64_t n = n0 + j;
#pragma unroll
            for (int e = 0; e < VK; ++e) {
                if (k + e < g.K) {
                    const int64_t bi = g.b_col ? n * g.ldb + k + e : (k + e) * g.ldb + n;
                    acc[j] = fmaf(a[e], elem_f32<AB_TYPE>(B, bi), acc[j]);
                }
            }
        }
    }
    // sum over the wavefront's 64 lanes
#pragma unroll
    for (int j = 0; j < kMaxSliver; ++j) {
        if (j >= nrem)
            break;
        float v = acc[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            v += __shfl_xor(v, off, 64);
        acc[j] = v;
    }
    if (lane < nrem) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxSliver; ++j)
            if (j == lane)
                v = acc[j];
        const int64_t n = n0 + lane;
        store_c(g, b, m, n, epilogue_value(g, b, m, n, v));
    }
}

} // namespace

hipError_t launch_sliver(const GemmArgs &g, int64_t n0, int32_t nrem, hipStream_t stream)
{
    const dim3 grid((unsigned)((g.M + kSliverThreads / 64 - 1) / (kSliverThreads / 64)),
                    (unsigned)g.sched.batch),
        block(kSliverThreads);
    if (g.ab_type == DT_BF16)
        hipLaunchKernelGGL((gemm_sliver_kernel<DT_BF16>), grid, block, 0, stream, g, n0, nrem);
    else if (g.ab_type == DT_F16)
        hipLaunchKernelGGL((gemm_sliver_kernel<DT_F16>), grid, block, 0, stream, g, n0, nrem);
    else
        hipLaunchKernelGGL((gemm_sliver_kernel<DT_F32>), grid, block, 0, stream, g, n0, nrem);
    return hipGetLastError();
}

} // namespace dg
