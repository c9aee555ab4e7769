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
//     c ^ (r mod 8) (XOR swizzle), so both the stores and the fragment
//     reads below touch 8 different 16-byte bank groups per 8 lanes;
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

// 8 bf16 at p[off .. off+7], element j present iff line_ok && first+j < limit.
__device__ __forceinline__ uint4 load_chunk_masked(const uint16_t *p, int64_t off, bool line_ok,
                                                   int64_t first, int64_t limit)
{
    if (line_ok && first + 8 <= limit)
        return *(const uint4 *)(p + off);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (line_ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (first + j < limit)
                w[j / 2] |= (uint32_t)p[off + j] << (16 * (j % 2));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
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

    uint4 ra[ACH], rb[BCH];

    auto load_tiles = [&](int64_t k0) {
        const int64_t gk = k0 + kc * 8;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int64_t gm = m0 + r0 + i * ROWS_PER_PASS;
            ra[i] = load_chunk_masked(A, gm * lda + gk, gm < M, gk, ke);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int64_t gn = n0 + r0 + i * ROWS_PER_PASS;
            rb[i] = load_chunk_masked(B, gn * ldb + gk, gn < N, gk, ke);
        }
    };

    auto store_tiles = [&](int st) {
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int r = r0 + i * ROWS_PER_PASS;
            As[st * A_STAGE + r * 8 + (kc ^ (r & 7))] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int r = r0 + i * ROWS_PER_PASS;
            Bs[st * B_STAGE + r * 8 + (kc ^ (r & 7))] = rb[i];
        }
    };

    const int frag_row = lane & 31;       // row of A / column of B this lane feeds
    const int frag_half = lane >> 5;      // which 8 of the 16 k of one MFMA step
    const int swz = lane & 7;             // == frag row mod 8 (wave tiles are 32-aligned)

    auto compute = [&](int st) {
        const uint4 *as = As + st * A_STAGE + (wm * TM + frag_row) * 8;
        const uint4 *bs = Bs + st * B_STAGE + (wn * TN + frag_row) * 8;
#pragma unroll
        for (int ks = 0; ks < MBK / 16; ++ks) {
            const int c = (ks * 2 + frag_half) ^ swz;
            bf16x8_t af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t, as[i * 32 * 8 + c]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = __builtin_bit_cast(bf16x8_t, bs[j * 32 * 8 + c]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };

    const int64_t nk = (ke > kb) ? (ke - kb + MBK - 1) / MBK : 0;
    if (g.alpha != 0.0f && nk > 0) {
        load_tiles(kb);
        store_tiles(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int st = (int)(kt & 1);
            if (kt + 1 < nk)
                load_tiles(kb + (kt + 1) * MBK);
            compute(st);
            if (kt + 1 < nk)
                store_tiles(st ^ 1);
            __syncthreads();
        }
    }

    // Output layout of a 32x32 block: lane l, register v holds
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t gn = n0 + wn * TN + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t gm = m0 + wm * TM + i * 32 + 8 * (v / 4) + 4 * frag_half + (v % 4);
                if (gm < M && gn < N)
                    write_result(g, tc.b, tc.s, gm, gn, acc[i][j][v]);
            }
        }
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
