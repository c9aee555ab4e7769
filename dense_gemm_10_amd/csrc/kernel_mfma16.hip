// bf16 and fp16 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16 and
// its fp16 twin v_mfma_f32_32x32x16_f16), fp32 accumulation.  The two
// element types share every byte of the data path (loads, LDS layout,
// fragments, epilogue); only the MFMA instruction differs.
//
// The structure is the tiled blocked GEMM of "GEMM Kernel Optimization"
// (Core Technique: one workgroup per BM x BN output tile, K walked in
// BK chunks, fp32 accumulators, cast on store) with the matrix-core inner
// loop of its "Tensor Core Utilization" section and the three tiling levels
// of "La GEMM, de zero a cuBLAS" (workgroup tile in LDS, wave tile in
// registers, 32 x 32 x 16 MFMA fragments).  The multi-stage ring below is
// the double buffering of that page's section 2.8 taken further.
//
// Operands: A row-major (M x K) and B column-major (K x N), i.e. both with
// K contiguous, which is the order an MFMA lane consumes: lane l supplies 8
// consecutive k of row (l mod 32) of A and of column (l mod 32) of B.
//
// Data path:
//   global -> LDS: direct DMA (global_load_lds_dwordx4): each instruction
//     moves 64 x 16 bytes, lane l's 16 bytes landing at LDS address
//     M0 + 16 l, without passing through registers.  A K tile (BK = 32 or
//     64) of A and of B is a "stage"; NSTAGE stages form a ring and the
//     loads of tile t + NSTAGE - 1 are issued while tile t is multiplied, so
//     each load has NSTAGE - 1 tiles of MFMA work to arrive in.  With
//     BK = 64 a row of a stage is a whole 128-byte line of A or B; 64-byte
//     half lines were measured to cap the L2 -> CU stream at about 80 % of
//     what whole lines reach.
//   LDS layout: a stage row (one row of A, or one column of B) is BK * 2
//     bytes = CPR chunks of 8 16-bit elements; logical chunk c of row r is stored at
//     slot c ^ ((r / (16 / CPR)) mod CPR).  The LDS serves a 128-bit access
//     16 lanes at a time over 256 bytes of banks; 16 lanes reading one
//     logical chunk of 16 consecutive rows then hit 16 different 16-byte
//     bank groups.  The DMA lanes are assigned so that consecutive lanes
//     fill consecutive slots: lane l loads the global chunk that belongs in
//     slot l.
//   LDS -> registers: ds_read_b128 fragments, BK / 16 k-steps per stage;
//   MFMA: each wavefront owns a TM x TN wave tile = FM x FN blocks of
//     32 x 32, accumulated in FM*FN*16 fp32 registers per lane.
// The DMA is issued through inline assembly so that the compiler does not
// serialise it: vector-memory loads of a wave complete in order, so waiting
// until at most (NSTAGE - 2) tiles' loads are outstanding (s_waitcnt
// vmcnt), then one workgroup barrier, makes a stage readable and the stage
// read in the previous iteration writable.
//
// A partial last K tile (K not a multiple of BK) is loaded first, through
// registers with a K mask, so the steady-state loop is uniform.  Rows past
// M (or N) are clamped to the last row: the loads stay inside the matrix
// and those rows only feed outputs that are never stored.
//
// Requirements checked on the host: bf16 or fp16 A (row-major) and B
// (column-major), of one type; 16-byte aligned base pointers; lda, ldb and the batch strides
// multiples of 8 elements; BM * lda and BN * ldb small enough for 32-bit
// byte offsets inside a tile.
#include "epilogue.hpp"
#include "launch.hpp"

namespace dg {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Fragment type of element type T, and the 32 x 32 x 16 MFMA on it.
template <int T> struct frag_of { using type = bf16x8_t; };
template <> struct frag_of<DT_F16> { using type = f16x8_t; };

__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(f16x8_t a, f16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}


// s_waitcnt immediate: wait until at most n vector-memory loads of this
// wave are outstanding and all its LDS operations have completed (expcnt
// left unconstrained).
constexpr int vm_lgkm0_imm(int n)
{
    return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (0 << 8);
}

// A value that is the same in every lane, moved to scalar registers (the
// compiler cannot prove uniformity of results of 64-bit divisions).
__device__ __forceinline__ int64_t uniform_i64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ const void *uniform_ptr(const void *p)
{
    return (const void *)uniform_i64((int64_t)(uintptr_t)p);
}

// One DMA instruction: 16 bytes per lane from base + voff (bytes) into LDS
// at lds_addr + 16 * lane.  lds_addr must be wave-uniform.
__device__ __forceinline__ void dma_16(const void *base, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}

// Cache policy of the tile loads.  The pages suggest evict-first for A and
// evict-last for B ("Skill: Write a Triton GEMM Kernel", Kernel design
// rules).  CDNA4's global loads carry no evict-last bit; their
// evict-first counterpart is the non-temporal bit `nt` (streaming
// replacement in the L2).  Building with -DDG_LOAD_POLICY_A=nt (or _B)
// appends that bit to the A (or B) tile loads.  Off by default: measured on
// the 4096^3 bf16 GEMM, the L2 hit rate stays at 0.80 either way and the
// kernel runs 6 to 12 % slower (22 to 31 % on the ragged 4095 x 4097 x 1000
// GEMM).
#if defined(DG_LOAD_POLICY_A) || defined(DG_LOAD_POLICY_B)
#define DG_LOAD_POLICY 1
#define DG_STR2(x) #x
#define DG_STR(x) DG_STR2(x)
#ifndef DG_LOAD_POLICY_A
#define DG_LOAD_POLICY_A
#endif
#ifndef DG_LOAD_POLICY_B
#define DG_LOAD_POLICY_B
#endif
__device__ __forceinline__ void dma_16_policy(bool a, const void *base, uint32_t voff,
                                              uint32_t lds_addr)
{
    if (a)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 "
                     DG_STR(DG_LOAD_POLICY_A)
                     :
                     : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 "
                     DG_STR(DG_LOAD_POLICY_B)
                     :
                     : "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                     : "memory", "m0");
}
#endif

// 8 16-bit elements of one row at k = k_first .. k_first+7, zero for k >= ke (the
// K-boundary mask of a partial K tile).  `row` points at k = 0 of the row;
// ke >= 1.  A chunk wholly inside the range is one 16-byte load (the row's
// chunks are 16-byte aligned: lda is a multiple of 8 and the base
// aligned), one wholly past it is zero without a load, and only the chunk
// that straddles ke is read element by element (with the index clamped to
// ke - 1, so every load stays inside the row).
__device__ __forceinline__ uint4 load_chunk_tail(const uint16_t *row, int64_t k_first,
                                                 int64_t ke)
{
    if (k_first + 8 <= ke)
        return *(const uint4 *)(row + k_first);
    if (k_first >= ke)
        return make_uint4(0u, 0u, 0u, 0u);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = k_first + j;
        const uint32_t v = row[k < ke ? k : ke - 1];
        w[j / 2] |= (k < ke ? v : 0u) << (16 * (j % 2));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Swizzle key of stage row r for CPR 16-byte chunks per row: rows that
// share a 256-byte bank line get different keys, and so do the 16 rows one
// 16-lane group of a fragment read touches.
template <int CPR>
__device__ __forceinline__ int swizzle_key(int r)
{
    return (r / (16 / CPR)) % CPR;
}

// LDS of one workgroup: the stage ring, or the epilogue's chunk and bias
// when those are larger (short rings of wide tiles).
constexpr int mfma16_lds_bytes(int BM, int BN, int NS, int BK)
{
    return NS * (BM + BN) * (BK / 8) * 16 > epilogue_lds_bytes(BN)
               ? NS * (BM + BN) * (BK / 8) * 16
               : epilogue_lds_bytes(BN);
}

// Workgroups one CU holds at once: LDS allows 160 KB / mfma16_lds_bytes,
// and registers 512 per SIMD lane over one wave's (each workgroup puts one
// wave on each SIMD).  A wave's registers are its BM*BN/256 fp32
// accumulators plus about as many again for fragments, addresses and the
// epilogue, so a 256 x 256 tile gets one workgroup per CU, 256 x 128 and
// 128 x 256 two and 128 x 128 four; the kernels are compiled to that
// register budget (amdgpu_waves_per_eu) and the planner sizes full waves
// of stream-K and split-K by it.
constexpr int mfma16_per_cu(int BM, int BN, int NS, int BK)
{
    const int by_lds = 160 * 1024 / mfma16_lds_bytes(BM, BN, NS, BK);
    const int by_regs = 4 * 128 * 128 / (BM * BN);
    return by_lds < by_regs ? by_lds : by_regs;
}

// One output tile (or, for stream-K, one K range of it): K loop over
// [kb, ke) and the epilogue, or the raw fp32 accumulators written to `part`
// (a BM x BN row-major slot) when `part` is not null.
template <int T, int BM, int BN, int WM, int WN, int kStages, int MBK>
__device__ __forceinline__ void mfma16_tile(const GemmArgs &g, TileCoord tc, int64_t kb,
                                            int64_t ke, float *part, uint4 *lds)
{
    using frag_t = typename frag_of<T>::type;
    constexpr int NT = 64 * WM * WN;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;    // wave tile
    constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 blocks per wave
    constexpr int CPR = MBK / 8;                 // 16-byte chunks per stage row
    constexpr int KS = MBK / 16;                 // MFMA k-steps per stage
    constexpr int RPI = 64 / CPR;                // stage rows per DMA instruction
    constexpr int ROWS = BM + BN;                // stage rows: A rows, then B columns
    constexpr int GROUPS = ROWS / RPI;           // DMA instructions per stage
    constexpr int LPW = GROUPS / NW;             // ... per wave
    constexpr int STAGE_SLOTS = ROWS * CPR;      // 16-byte slots per stage
    constexpr int D = kStages - 1;               // prefetch distance (tiles)
    static_assert((D - 1) * LPW <= 63, "loads left in flight fit the vmcnt counter");
    static_assert(MBK == 32 || MBK == 64, "stage K width");
    static_assert(KS % 2 == 0, "fragment sets alternate per k-step");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BM % RPI == 0 && BN % RPI == 0 && GROUPS % NW == 0, "DMA split");

    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)lds;

    tc.b = uniform_i64(tc.b);
    tc.s = __builtin_amdgcn_readfirstlane(tc.s);
    tc.pid_m = __builtin_amdgcn_readfirstlane(tc.pid_m);
    tc.pid_n = __builtin_amdgcn_readfirstlane(tc.pid_n);
    const int64_t m0 = (int64_t)tc.pid_m * BM;
    const int64_t n0 = (int64_t)tc.pid_n * BN;
    kb = uniform_i64(kb);
    ke = uniform_i64(ke);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int wm = wave / WN, wn = wave % WN;
    const int64_t M = g.M, N = g.N, lda = g.lda, ldb = g.ldb;
    const uint16_t *A_tile = (const uint16_t *)g.A + tc.b * g.sa + m0 * lda;
    const uint16_t *B_tile = (const uint16_t *)g.B + tc.b * g.sb + n0 * ldb;

    // This lane's DMA sources: group q = wave * LPW + i covers stage rows
    // RPI q .. RPI q + RPI - 1 (A rows first, then B columns); lane l fills
    // slot 64q + l = (row RPI q + l / CPR, physical chunk l % CPR), i.e.
    // logical chunk (l % CPR) ^ key(row).  Byte offsets are relative to the
    // tile's first row and K position; rows past the matrix are clamped.
    uint32_t voff[LPW];
    bool from_a[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = wave * LPW + i;
        const int srow = q * RPI + lane / CPR;                     // stage row
        const int c = (lane % CPR) ^ swizzle_key<CPR>(srow);       // logical chunk
        from_a[i] = q * RPI < BM;                     // per group, hence wave-uniform
        int64_t r = from_a[i] ? srow : srow - BM;     // row inside the A / B tile
        const int64_t lim = from_a[i] ? M - m0 : N - n0;
        r = r < lim ? r : lim - 1;
        voff[i] = (uint32_t)((r * (from_a[i] ? lda : ldb) + c * 8) * 2);
    }

    // K position of virtual tile v: a partial tile (if any) comes first.
    const int64_t klen = ke > kb ? ke - kb : 0;
    const int64_t nfull = klen / MBK;
    const bool tail = (klen % MBK) != 0;
    const int64_t ntiles = nfull + (tail ? 1 : 0);
    auto tile_k0 = [&](int64_t v) -> int64_t {
        if (tail)
            return v == 0 ? kb + nfull * MBK : kb + (v - 1) * MBK;
        return kb + v * MBK;
    };

    // DMA instruction i (of LPW) of full tile v into its stage.
    auto issue_dma_one = [&](int64_t v, int i) {
        const int64_t k0 = tile_k0(v);
        const uint32_t stage_addr = lds_base + (uint32_t)((v % kStages) * STAGE_SLOTS * 16);
        const int q = wave * LPW + i;
#ifdef DG_LOAD_POLICY
        dma_16_policy(from_a[i], uniform_ptr((from_a[i] ? A_tile : B_tile) + k0), voff[i],
                      stage_addr + (uint32_t)(q * 64 * 16));
#else
        dma_16(uniform_ptr((from_a[i] ? A_tile : B_tile) + k0), voff[i],
               stage_addr + (uint32_t)(q * 64 * 16));
#endif
    };
    auto issue_dma = [&](int64_t v) {
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            issue_dma_one(v, i);
    };

    // The partial tile: same slots as the DMA, through registers, with the
    // K mask.
    auto load_tail = [&](int64_t v) {
        const int64_t k0 = tile_k0(v);
        uint4 *stage = lds + (v % kStages) * STAGE_SLOTS;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int q = wave * LPW + i;
            const int srow = q * RPI + lane / CPR;
            const int c = (lane % CPR) ^ swizzle_key<CPR>(srow);
            const uint16_t *rowp = (const uint16_t *)((const char *)(from_a[i] ? A_tile : B_tile) +
                                                      voff[i]) - c * 8;
            stage[q * 64 + lane] = load_chunk_tail(rowp, k0 + c * 8, ke);
        }
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[i][j][v] = 0.0f;

    const int frag_row = lane & 31;       // row of A / column of B this lane feeds
    const int frag_half = lane >> 5;      // which 8 of the 16 k of one MFMA step
    const int swz = swizzle_key<CPR>(frag_row);   // key of every fragment row (period 16)

    // Fragments of k-step ks (0 .. KS-1) of a stage.
    auto load_frags = [&](int st, int ks, frag_t *af, frag_t *bf) {
        const uint4 *as = lds + st * STAGE_SLOTS + (wm * TM + frag_row) * CPR;
        const uint4 *bs = lds + st * STAGE_SLOTS + (BM + wn * TN + frag_row) * CPR;
        const int c = (ks * 2 + frag_half) ^ swz;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = __builtin_bit_cast(frag_t, as[i * 32 * CPR + c]);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bf[j] = __builtin_bit_cast(frag_t, bs[j * 32 * CPR + c]);
    };

    auto mfma_step = [&](const frag_t *af, const frag_t *bf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mfma_32x32x16(af[i], bf[j], acc[i][j]);
    };

    // Two fragment register sets, alternating per k-step; fa[1]/fb[1]
    // carry the last k-step of a stage into the next iteration, whose MFMAs
    // run after the barrier while the new stage's first fragments are read.
    frag_t fa[2][FM], fb[2][FN];

    // One stage, as KS k-steps of FM * FN fenced slots.  Slot n of k-step ks
    // issues the MFMA of block n on the previous k-step's fragments and,
    // in the first FM + FN slots, the read of one fragment of k-step ks, so
    // the LDS reads are spread over the matrix work instead of bunched in
    // front of it (or sunk next to their first use, where the compiler puts
    // them when left alone).  In the steady state the DMA of a later tile
    // is spread over the first DMA_STEPS k-steps (one instruction after
    // every MFMA_PER_DMA slots): DMA instructions closer than about two
    // MFMAs apart stall the in-order wave on the memory pipe while the
    // matrix pipe runs dry, and with a 2-stage ring the loads must still
    // start in the first half of the iteration to arrive before the next
    // one (measured: first quarter 15 % slower, whole stage 23 % slower).
    constexpr int DMA_STEPS = kStages == 2 ? KS / 2 : KS;
    static_assert(DMA_STEPS >= 1 && DMA_STEPS <= KS, "DMA window inside the stage");
    constexpr int DMA_WINDOW = DMA_STEPS * FM * FN;
    constexpr int MFMA_PER_DMA = DMA_WINDOW / LPW > 0 ? DMA_WINDOW / LPW : 1;
    static_assert(FM + FN <= FM * FN, "fragment reads fit in the slots");
    auto stage_body = [&](int st, bool dma, int64_t v_dma) {
        const uint4 *as = lds + st * STAGE_SLOTS + (wm * TM + frag_row) * CPR;
        const uint4 *bs = lds + st * STAGE_SLOTS + (BM + wn * TN + frag_row) * CPR;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1, prev = cur ^ 1;
            const int c = (ks * 2 + frag_half) ^ swz;
#pragma unroll
            for (int n = 0; n < FM * FN; ++n) {
                if (n < FM)
                    fa[cur][n] = __builtin_bit_cast(frag_t, as[n * 32 * CPR + c]);
                else if (n < FM + FN)
                    fb[cur][n - FM] = __builtin_bit_cast(frag_t, bs[(n - FM) * 32 * CPR + c]);
                const int i = n / FN, j = n % FN;
                acc[i][j] = mfma_32x32x16(fa[prev][i], fb[prev][j], acc[i][j]);
                const int d = ks * FM * FN + n;
                if (dma && (d % MFMA_PER_DMA) == MFMA_PER_DMA - 1 && d / MFMA_PER_DMA < LPW)
                    issue_dma_one(v_dma, d / MFMA_PER_DMA);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Barrier that the compiler may not move LDS accesses across.  It is
    // always preceded by a wait for this wave's LDS reads (lgkmcnt 0), so a
    // stage that any wave still reads is never the target of a DMA issued
    // after the barrier.
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    if (g.alpha != 0.0f && ntiles > 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[1][i] = frag_t{};
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[1][j] = frag_t{};
        // prologue: tiles 0 .. D-1
        for (int64_t v = 0; v < D && v < ntiles; ++v) {
            if (v == 0 && tail)
                load_tail(0);
            else
                issue_dma(v);
        }
        if (tail)
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the register-path LDS writes
        int64_t v = 0;
        // steady state: D-1 later tiles stay in flight while tile v is used
        for (; v + D < ntiles; ++v) {
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm((D - 1) * LPW));
            barrier();
            stage_body((int)(v % kStages), true, v + D);
        }
        // drain
        for (; v < ntiles; ++v) {
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
            barrier();
            stage_body((int)(v % kStages), false, 0);
        }
        mfma_step(fa[1], fb[1]);   // last k-step of the last stage
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
        barrier();
    }

    // the epilogue keeps within the kernel's register budget
    constexpr int REGS = 512 / mfma16_per_cu(BM, BN, kStages, MBK);
    if (part)
        tile_epilogue_rows<BM, BN, WM, WN, true, DT_F32, REGS>(g, (char *)part, BN, BM, BN, n0,
                                                               (float *)lds, acc);
    else
        tile_epilogue<BM, BN, WM, WN, REGS>(g, tc, (float *)lds, m0, n0, acc);
}

// Data-parallel launches give each program one tile (or split-K slice).
// Stream-K launches give programs [0, dp_tiles) one whole tile each and the
// others one K slice of a tail tile, written as a raw fp32 partial that the
// fix-up kernel adds up.
template <int T, int BM, int BN, int WM, int WN, int kStages, int MBK>
__device__ __forceinline__ void mfma16_program(const GemmArgs &g, uint4 *lds)
{
    const StreamK &sk = g.sk;
    const int64_t pid = blockIdx.x;
    TileCoord tc;
    int64_t kb, ke;
    float *part = nullptr;
    if (sk.tail_tiles == 0) {
        tc = decode_program(pid, g.sched);
        split_range(g, tc.s, kb, ke);
    } else if (pid < sk.dp_tiles) {
        tc = decode_tile(g.sched.xcd_remap ? xcd_remap(pid, sk.dp_tiles) : pid, g.sched);
        kb = 0;
        ke = g.K;
    } else {
        // dp_tiles is a multiple of 8, so the remap keeps each program on
        // its XCD; an XCD's programs then share slices and tile rows.
        const int64_t n = sk.tail_tiles * sk.tail_splits;
        const int64_t i = g.sched.xcd_remap ? xcd_remap(pid - sk.dp_tiles, n) : pid - sk.dp_tiles;
        const int64_t slice = i / sk.tail_tiles, r = i % sk.tail_tiles;
        tc = decode_tile(sk.dp_tiles + r, g.sched);
        kb = slice * sk.k_per_split;
        ke = kb + sk.k_per_split < g.K ? kb + sk.k_per_split : g.K;
        part = g.sk_parts + (r * sk.tail_splits + slice) * (int64_t)(BM * BN);
    }
    mfma16_tile<T, BM, BN, WM, WN, kStages, MBK>(g, tc, kb, ke, part, lds);
}

// One kernel name per element type, so that traces tell them apart.
template <int BM, int BN, int WM, int WN, int kStages, int MBK>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(mfma16_per_cu(BM, BN, kStages, MBK))))
void gemm_mfma_bf16_kernel(GemmArgs g)
{
    extern __shared__ uint4 lds[];
    mfma16_program<DT_BF16, BM, BN, WM, WN, kStages, MBK>(g, lds);
}

template <int BM, int BN, int WM, int WN, int kStages, int MBK>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(mfma16_per_cu(BM, BN, kStages, MBK))))
void gemm_mfma_f16_kernel(GemmArgs g)
{
    extern __shared__ uint4 lds[];
    mfma16_program<DT_F16, BM, BN, WM, WN, kStages, MBK>(g, lds);
}

template <int T, int BM, int BN, int WM, int WN, int NS, int BK>
hipError_t launch_one(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const size_t lds_bytes = (size_t)mfma16_lds_bytes(BM, BN, NS, BK);
    const dim3 grid((unsigned)p.programs), block(64 * WM * WN);
    if constexpr (T == DT_F16)
        hipLaunchKernelGGL((gemm_mfma_f16_kernel<BM, BN, WM, WN, NS, BK>), grid, block, lds_bytes,
                           stream, g);
    else
        hipLaunchKernelGGL((gemm_mfma_bf16_kernel<BM, BN, WM, WN, NS, BK>), grid, block, lds_bytes,
                           stream, g);
    return hipGetLastError();
}

} // namespace

// variant index -> instantiation (BM x BN tile, WM x WN wavefronts, ring
// depth); the last field is mfma16_per_cu of the instantiation.
// Entries 0 and 1 are the large and small tiles of the automatic choice:
// 256 x 256 with whole-line (BK = 64) stages in a 2-stage ring, and
// 128 x 128 with BK = 32 in a 4-stage ring (64 KB of LDS, two workgroups
// per CU).  The others are selectable by name for sweeps.  The fp16 table
// holds the two tiles of the automatic choice.
#define DG_TILE16(T, BM, BN, BK, NS, V) \
    {BM, BN, BK, 256, V, "mfma_" #T "_" #BM "x" #BN "x" #BK "_w2x2_s" #NS, mfma16_per_cu(BM, BN, NS, BK)}
const TileConfig kMfmaBf16Tiles[] = {
    DG_TILE16(bf16, 256, 256, 64, 2, 5),
    DG_TILE16(bf16, 128, 128, 32, 4, 1),
    DG_TILE16(bf16, 256, 256, 32, 4, 0),
    DG_TILE16(bf16, 256, 128, 32, 4, 2),
    DG_TILE16(bf16, 256, 128, 32, 3, 3),
    DG_TILE16(bf16, 128, 256, 32, 3, 4),
    DG_TILE16(bf16, 128, 128, 64, 3, 6),
    DG_TILE16(bf16, 256, 128, 64, 3, 7),
    DG_TILE16(bf16, 128, 256, 32, 2, 8),
    DG_TILE16(bf16, 128, 128, 32, 2, 9),
};
const int kNumMfmaBf16Tiles = 10;

const TileConfig kMfmaF16Tiles[] = {
    DG_TILE16(f16, 256, 256, 64, 2, 5),
    DG_TILE16(f16, 128, 128, 32, 4, 1),
};
#undef DG_TILE16
const int kNumMfmaF16Tiles = 2;

hipError_t launch_mfma16(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    if (g.ab_type == DT_F16) {
        switch (p.tile.variant) {
        case 1: return launch_one<DT_F16, 128, 128, 2, 2, 4, 32>(g, p, stream);
        case 5: return launch_one<DT_F16, 256, 256, 2, 2, 2, 64>(g, p, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.tile.variant) {
    case 0: return launch_one<DT_BF16, 256, 256, 2, 2, 4, 32>(g, p, stream);
    case 1: return launch_one<DT_BF16, 128, 128, 2, 2, 4, 32>(g, p, stream);
    case 2: return launch_one<DT_BF16, 256, 128, 2, 2, 4, 32>(g, p, stream);
    case 3: return launch_one<DT_BF16, 256, 128, 2, 2, 3, 32>(g, p, stream);
    case 4: return launch_one<DT_BF16, 128, 256, 2, 2, 3, 32>(g, p, stream);
    case 5: return launch_one<DT_BF16, 256, 256, 2, 2, 2, 64>(g, p, stream);
    case 6: return launch_one<DT_BF16, 128, 128, 2, 2, 3, 64>(g, p, stream);
    case 7: return launch_one<DT_BF16, 256, 128, 2, 2, 3, 64>(g, p, stream);
    case 8: return launch_one<DT_BF16, 128, 256, 2, 2, 2, 32>(g, p, stream);
    case 9: return launch_one<DT_BF16, 128, 128, 2, 2, 2, 32>(g, p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace dg
