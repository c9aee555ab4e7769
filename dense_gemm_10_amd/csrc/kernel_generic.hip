// Generic LDS-tiled GEMM: every dtype pair, every operand order, any
// leading dimension / alignment / batch stride, masked edges, split-K.
//
// This is the shared-memory tiling of "La GEMM, de zero a cuBLAS" section
// 2.4 (cooperative tile loads with zero fill outside the matrix, barrier,
// inner product over the staged tile, barrier) widened to a 4 x 4
// register block per thread (section 2.6).  It is the correctness fallback
// for shapes and layouts the specialised kernels do not take; fast paths
// live in the VALU and MFMA kernel files.
//
// Tile 64 x 64 x 16, 256 threads.  Thread (tx, ty) owns rows ty + 16 i and
// columns tx + 16 j, i, j < 4, so a wavefront reads 4 distinct A words
// (broadcast) and 16 consecutive B words per LDS access.  Global loads walk
// the operand's contiguous dimension with consecutive threads (coalescing,
// section 2.3).  Loads are masked on the row / column index and on the K
// range of the program's split ("Skill: Write a Triton GEMM Kernel",
// Required reasoning process step 5): masked elements read as 0.
#include "launch.hpp"

namespace dg {

namespace {

constexpr int GBM = 64, GBN = 64, GBK = 16, GTHREADS = 256;

template <int AB_TYPE>
__global__ __launch_bounds__(GTHREADS) void gemm_generic_kernel(GemmArgs g)
{
    __shared__ float As[GBK][GBM + 1];
    __shared__ float Bs[GBK][GBN + 1];

    const TileCoord tc = decode_program(blockIdx.x, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * GBM;
    const int64_t n0 = (int64_t)tc.pid_n * GBN;
    int64_t kb, ke;
    split_range(g, tc.s, kb, ke);

    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.0f;

    if (g.alpha != 0.0f) {
        const int64_t abase = tc.b * g.sa;
        const int64_t bbase = tc.b * g.sb;
        for (int64_t k0 = kb; k0 < ke; k0 += GBK) {
            // A tile: 64 rows x 16 k.  Consecutive threads follow the
            // contiguous dimension of A.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int idx = tid + GTHREADS * e;
                int mm, kk;
                if (g.a_col) { mm = idx % GBM; kk = idx / GBM; }
                else         { kk = idx % GBK; mm = idx / GBK; }
                const int64_t gm = m0 + mm, gk = k0 + kk;
                float v = 0.0f;
                if (gm < g.M && gk < ke)
                    v = load_as_f32(g.A, AB_TYPE, abase + elem_offset(g.a_col, g.lda, gm, gk));
                As[kk][mm] = v;
            }
            // B tile: 16 k x 64 columns.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int idx = tid + GTHREADS * e;
                int nn, kk;
                if (g.b_col) { kk = idx % GBK; nn = idx / GBK; }
                else         { nn = idx % GBN; kk = idx / GBN; }
                const int64_t gn = n0 + nn, gk = k0 + kk;
                float v = 0.0f;
                if (gn < g.N && gk < ke)
                    v = load_as_f32(g.B, AB_TYPE, bbase + elem_offset(g.b_col, g.ldb, gk, gn));
                Bs[kk][nn] = v;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < GBK; ++k) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = As[k][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = Bs[k][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
    }

    // Store masked on M and N.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gm = m0 + ty + 16 * i;
        if (gm >= g.M)
            continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gn = n0 + tx + 16 * j;
            if (gn < g.N)
                write_result(g, tc.b, tc.s, gm, gn, acc[i][j]);
        }
    }
}

// p[0] + p[stride] + ... + p[(count - 1) * stride], added left to right (a
// fixed order, so the result is reproducible), with the loads of up to
// eight partials issued before their additions: a loop of dependent
// load-add pairs waits one memory latency per partial.
template <typename V>
__device__ __forceinline__ void add_to(V &sum, const V &v);
template <>
__device__ __forceinline__ void add_to<float>(float &sum, const float &v) { sum += v; }
template <>
__device__ __forceinline__ void add_to<float4>(float4 &sum, const float4 &v)
{
    sum.x += v.x;
    sum.y += v.y;
    sum.z += v.z;
    sum.w += v.w;
}

template <typename V>
__device__ __forceinline__ V sum_partials(const float *p, int64_t stride, int64_t count)
{
    V sum{};
    int64_t s = 0;
    for (; s + 8 <= count; s += 8) {
        V v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = *(const V *)(p + (s + j) * stride);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            add_to(sum, v[j]);
    }
    if (s + 4 <= count) {
        V v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = *(const V *)(p + (s + j) * stride);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            add_to(sum, v[j]);
        s += 4;
    }
    for (; s < count; ++s)
        add_to(sum, *(const V *)(p + s * stride));
    return sum;
}

// Split-K reduction: for each output element, sum the S partials in split
// order (a fixed order, so the result is reproducible), then apply the
// epilogue exactly once.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int32_t splits)
{
    const int64_t total = g.sched.batch * g.M * g.N;
    const int64_t plane = total;                  // one split's partials
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const float sum = sum_partials<float>(g.ws + e, plane, splits);
        const int64_t n = e % g.N;
        const int64_t bm = e / g.N;
        const int64_t m = bm % g.M;
        const int64_t b = bm / g.M;
        store_c(g, b, m, n, epilogue_value(g, b, m, n, sum));
    }
}

// The same reduction, four consecutive outputs of one row per thread, when
// N is a multiple of 4 and the batch's outputs fit 32-bit indices: one
// 16-byte read per split and per thread, and 32-bit row / column math.
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(GemmArgs g, int32_t splits)
{
    const uint32_t total = (uint32_t)(g.sched.batch * g.M * g.N);
    const uint32_t N = (uint32_t)g.N, M = (uint32_t)g.M;
    for (uint32_t e = (blockIdx.x * 256u + threadIdx.x) * 4u; e < total;
         e += gridDim.x * 1024u) {
        const float4 sum = sum_partials<float4>(g.ws + e, total, splits);
        const uint32_t row = e / N, n = e - row * N;
        const uint32_t b = row / M, m = row - b * M;
        const float acc[4] = {sum.x, sum.y, sum.z, sum.w};
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            v[j] = epilogue_value(g, b, m, n + j, acc[j]);
        // the four outputs are consecutive in a row-major C: one aligned
        // 8-byte (16-bit C) or 16-byte (fp32 C) non-temporal store
        const int64_t ci = (int64_t)b * g.sc + (int64_t)m * g.ldc + n;
        const int es = g.c_type == DT_F32 ? 4 : 2;
        char *dst = (char *)g.C + ci * es;
        if (!g.c_col && ((uintptr_t)dst & (uintptr_t)(4 * es - 1)) == 0) {
            if (g.c_type == DT_F32) {
                typedef float f32x4_nt __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store((f32x4_nt){v[0], v[1], v[2], v[3]}, (f32x4_nt *)dst);
            } else {
                typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
                uint32_t h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    h[j] = g.c_type == DT_F16 ? f32_to_f16(v[j]) : f32_to_bf16(v[j]);
                __builtin_nontemporal_store((u32x2_nt){h[0] | (h[1] << 16), h[2] | (h[3] << 16)},
                                            (u32x2_nt *)dst);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                store_c(g, b, m, n + j, v[j]);
        }
    }
}

// Stream-K fix-up: each tail tile left tail_splits fp32 partials in the
// workspace, one per K slice; add them in slice order (a fixed order, so
// the result is reproducible) and apply the epilogue once.
__global__ __launch_bounds__(256) void streamk_fixup_kernel(GemmArgs g, int32_t bm, int32_t bn)
{
    const int64_t area = (int64_t)bm * bn;                 // a multiple of 1024
    const int64_t per_tile = area / 1024;                  // blocks per tile, 4 outputs per thread
    const int64_t r = blockIdx.x / per_tile;
    const int64_t e0 = (blockIdx.x % per_tile) * 1024 + threadIdx.x * 4;
    const TileCoord tc = decode_tile(g.sk.dp_tiles + r, g.sched);
    const int64_t m0 = (int64_t)tc.pid_m * bm, n0 = (int64_t)tc.pid_n * bn;
    const int64_t row = e0 / bn, col = e0 % bn;            // 4 consecutive columns of one row
    const int64_t m = m0 + row;
    if (m >= g.M)
        return;
    const float *p = g.sk_parts + r * g.sk.tail_splits * area + e0;
    const float4 t = sum_partials<float4>(p, area, g.sk.tail_splits);
    const float sum[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + col + j;
        if (n < g.N)
            store_c(g, 0, m, n, epilogue_value(g, 0, m, n, sum[j]));
    }
}

} // namespace

const TileConfig kGenericTiles[] = {
    {GBM, GBN, GBK, GTHREADS, 0, "generic_64x64x16"},
};
const int kNumGenericTiles = 1;

hipError_t launch_generic(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.programs), block(GTHREADS);
    // A and B share a dtype (validated on the host).
    if (g.ab_type == DT_BF16)
        hipLaunchKernelGGL((gemm_generic_kernel<DT_BF16>), grid, block, 0, stream, g);
    else if (g.ab_type == DT_F16)
        hipLaunchKernelGGL((gemm_generic_kernel<DT_F16>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_generic_kernel<DT_F32>), grid, block, 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_streamk_fixup(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.fixup_blocks), block(256);
    hipLaunchKernelGGL(streamk_fixup_kernel, grid, block, 0, stream, g, p.tile.bm, p.tile.bn);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    dim3 grid((unsigned)p.reduce_blocks), block(256);
    if (reduce_by_four(g.N, g.sched.batch * g.M * g.N))
        hipLaunchKernelGGL(splitk_reduce4_kernel, grid, block, 0, stream, g, p.splits);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel, grid, block, 0, stream, g, p.splits);
    return hipGetLastError();
}

} // namespace dg
