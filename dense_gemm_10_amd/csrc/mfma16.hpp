// Templates of the bf16 and fp16 matrix-core GEMM, instantiated by the
// kernel_mfma16_*.hip files (one group of tile configurations each, so
// they compile in parallel); kernel_mfma16.hip holds the tile tables and
// the dispatch.
//
// bf16 and fp16 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16 and
// its fp16 twin v_mfma_f32_32x32x16_f16; the 256 x 256 tile uses the
// 16 x 16 x 32 shapes for every operand order, see mfma_16x16x32), fp32
// accumulation.  The two element types share every byte of the data path
// (loads, LDS layout, fragments, epilogue); only the MFMA instruction
// differs.
//
// The structure is the tiled blocked GEMM of "GEMM Kernel Optimization"
// (Core Technique: one workgroup per BM x BN output tile, K walked in
// BK chunks, fp32 accumulators, cast on store) with the matrix-core inner
// loop of its "Tensor Core Utilization" section and the three tiling levels
// of "La GEMM, de zero a cuBLAS" (workgroup tile in LDS, wave tile in
// registers, 32 x 32 x 16 MFMA fragments).  The multi-stage ring below is
// the double buffering of that page's section 2.8 taken further.
//
// Operands: an MFMA lane consumes 8 consecutive k of row (l mod 32) of A
// and of column (l mod 32) of B.  A row-major (M x K) and B column-major
// (K x N) have K contiguous and are staged as rows of K (below); a
// column-major A or row-major B (M or N contiguous, the orders of "Skill:
// Write a Triton GEMM Kernel", Inputs the agent should gather first, item 3)
// is staged as rows of M or N and transposed by the LDS reads (see
// mfma16_tile), so every layout runs on the matrix cores.
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
//   LDS -> registers: ds_read_b128 fragments, BK / 16 (BK / 32 with 16 x 16
//     blocks) k-steps per stage;
//   MFMA: each wavefront owns a TM x TN wave tile = FM x FN blocks of
//     32 x 32 (or 16 x 16), accumulated in TM*TN/64 fp32 registers per lane.
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
// Requirements checked on the host: bf16 or fp16 A and B of one type;
// 16-byte aligned base pointers; lda, ldb and the batch strides multiples
// of 8 elements; BM * lda and BN * ldb (or BK * lda, BK * ldb) small enough
// for 32-bit byte offsets inside a tile; an M- or N-contiguous operand only
// on the 256 x 256 and 128 x 128 tiles.
#pragma once
#include "epilogue.hpp"
#include "launch.hpp"
#include "sliver.hpp"

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

// The 16 x 16 x 32 shape: lane l holds A row l mod 16 (B column l mod 16),
// k = 8 (l / 16) .. + 7, and accumulates rows 4 (l / 16) .. + 3 of column
// l mod 16.  Under the chip's power limit it sustains about 13 % more
// than the 32 x 32 x 16 shape on the same data (a probe of both shapes fed
// from LDS: 1.64 against 1.45 PFLOP/s): half the accumulator register
// traffic per flop.
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32(f16x8_t a, f16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Accumulators of one MFMA block: 32 x 32 (16 per lane) or 16 x 16 (4).
template <int MS> struct acc_of { using type = f32x16_t; };
template <> struct acc_of<16> { using type = f32x4_t; };

template <typename F>
__device__ __forceinline__ f32x16_t mfma_block(F a, F b, f32x16_t c) { return mfma_32x32x16(a, b, c); }
template <typename F>
__device__ __forceinline__ f32x4_t mfma_block(F a, F b, f32x4_t c) { return mfma_16x16x32(a, b, c); }



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
constexpr int mfma16_lds_bytes(int BM, int BN, int NS, int BK, int MS = 32)
{
    return NS * (BM + BN) * (BK / 8) * 16 > epilogue_lds_bytes(BN, MS)
               ? NS * (BM + BN) * (BK / 8) * 16
               : epilogue_lds_bytes(BN, MS);
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

// Slot of logical 16-byte chunk c in k-row `k` of an operand staged with its
// M (or N) dimension contiguous: rows sit 64 bytes apart modulo the 256
// bytes of LDS banks, so the four k-rows one transposing read touches get
// four disjoint quarters of the banks; k-rows 8 apart (the other 16-lane
// group of the same half-wave in a 16 x 16 fragment read, or of the
// second half-wave in a 32 x 32 one) take the other pair of chunks.
__device__ __forceinline__ int mn_slot(int c, int k)
{
    return c ^ (4 * (k & 3)) ^ (2 * ((k >> 3) & 1));
}

// 8 16-bit elements at columns col .. col+7 of one row of an operand whose
// M (or N) dimension is contiguous, zero at columns >= ext (the M or N edge
// of the tile).  A chunk wholly inside is one 16-byte load; the chunk that
// straddles ext is read element by element with the index clamped to
// ext - 1, so no load leaves the row's valid part.
__device__ __forceinline__ uint4 load_chunk_cols(const uint16_t *row, int64_t col, int64_t ext)
{
    if (col + 8 <= ext)
        return *(const uint4 *)(row + col);
    if (col >= ext)
        return make_uint4(0u, 0u, 0u, 0u);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t c = col + j;
        const uint32_t v = row[c < ext ? c : ext - 1];
        w[j / 2] |= (c < ext ? v : 0u) << (16 * (j % 2));
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Fragment of an operand staged M- (or N-) contiguous: the 8 consecutive k
// of one row (column of B) that MFMA lane l consumes, gathered by two
// transposing LDS reads (ds_read_b64_tr_b16).  Within each group of 16
// lanes that instruction returns to lane i the (i mod 4)-th element of the
// 8-byte pieces addressed by lanes 4r + i / 4 of the group, r = 0 .. 3
// (measured on gfx950).  So lane 4r + q of group g addresses k-row
// kbase + r, columns 16 (g mod 2) + 4q .. +3 of the fragment, and lane
// l = 16g + i receives k-rows kbase .. kbase + 3 of column 16 (g mod 2) + i
// = l mod 32; kbase = 8 (l / 32) for the first read and 4 more for the
// second.  `addr0` is the lane's byte address for the first read; the
// second is 4 k-rows further.
template <typename frag_t, int ROW_BYTES>
__device__ __forceinline__ frag_t tr_fragment(uint32_t addr0)
{
    typedef __attribute__((address_space(3))) s16x4_t *lds_s4;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(uintptr_t)addr0);
    const s16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(uintptr_t)(addr0 + 4 * ROW_BYTES));
    const s16x8_t both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(frag_t, both);
}

// One output tile (or, for stream-K, one K range of it): K loop over
// [kb, ke) and the epilogue, or the raw fp32 accumulators written to `part`
// (a BM x BN row-major slot) when `part` is not null.
//
// AT / BT: A is stored M-contiguous (column-major) / B is stored
// N-contiguous (row-major).  Such an operand is staged as MBK k-rows of BM
// (BN) elements, loaded by the same DMA (whole 16-byte chunks along M or
// N, slots placed by mn_slot), and read into MFMA fragments by transposing
// LDS reads; the K-contiguous operands keep rows of K as above.  Columns
// past the M (N) edge are clamped to the last chunk that starts inside the
// edge; where the edge cuts a chunk, that chunk reaches up to 7 elements
// past the edge, inside the leading dimension for every k-row but the
// matrix's last, so a K range that ends at K loads its last K tile through
// registers with both masks.
template <int T, int BM, int BN, int WM, int WN, int kStages, int MBK, bool AT, bool BT,
          int MS = 32>
__device__ __forceinline__ void mfma16_tile(const GemmArgs &g, TileCoord tc, int64_t kb,
                                            int64_t ke, float *part, uint4 *lds)
{
    using frag_t = typename frag_of<T>::type;
    constexpr int NT = 64 * WM * WN;
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;    // wave tile
    constexpr int FM = TM / MS, FN = TN / MS;    // MS x MS MFMA blocks per wave
    constexpr int KD = MS == 32 ? 16 : 32;       // k of one MFMA
    constexpr int CPS = KD / 8;                  // 16-byte chunks of a fragment row per k-step
    constexpr int CPR = MBK / 8;                 // 16-byte chunks per stage row
    constexpr int KS = MBK / KD;                 // MFMA k-steps per stage
    using acc_t = typename acc_of<MS>::type;
    constexpr int NV = MS == 32 ? 16 : 4;        // accumulators per lane per block
    static_assert(MS == 32 || MS == 16, "MFMA block size");
    constexpr int RPI = 64 / CPR;                // stage rows per DMA instruction
    constexpr int ROWS = BM + BN;                // stage rows: A rows, then B columns
    constexpr int GROUPS = ROWS / RPI;           // DMA instructions per stage
    constexpr int A_GROUPS = BM / RPI;           // ... of A (the same count either layout)
    constexpr int LPW = GROUPS / NW;             // ... per wave
    constexpr int STAGE_SLOTS = ROWS * CPR;      // 16-byte slots per stage
    constexpr int D = kStages - 1;               // prefetch distance (tiles)
    constexpr int A_CPK = BM / 8, B_CPK = BN / 8;   // chunks per k-row, M-/N-contiguous
    static_assert((D - 1) * LPW <= 63, "loads left in flight fit the vmcnt counter");
    static_assert(MBK == 32 || MBK == 64, "stage K width");
    static_assert(KS % 2 == 0, "fragment sets alternate per k-step");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BM % RPI == 0 && BN % RPI == 0 && GROUPS % NW == 0, "DMA split");
    static_assert((!AT || (A_CPK >= 16 && 64 % A_CPK == 0)) &&
                  (!BT || (B_CPK >= 16 && 64 % B_CPK == 0)),
                  "M-/N-contiguous staging needs 128 or 256 elements per k-row");

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
    const int64_t a_ext = M - m0 < BM ? M - m0 : BM;   // valid rows of A / columns of B
    const int64_t b_ext = N - n0 < BN ? N - n0 : BN;
    // tile origin: row m0 (column n0) of a K-contiguous operand, column m0
    // (n0) of k-row 0 of an M- (N-) contiguous one
    const uint16_t *A_tile = (const uint16_t *)g.A + tc.b * g.sa + (AT ? m0 : m0 * lda);
    const uint16_t *B_tile = (const uint16_t *)g.B + tc.b * g.sb + (BT ? n0 : n0 * ldb);

    // This lane's DMA sources.  Group q = wave * LPW + i fills slots
    // 64q .. 64q + 63 of a stage (A's groups first, then B's); lane l fills
    // slot 64q + l.  K-contiguous operand: stage row RPI q + l / CPR (a row
    // of A or column of B, clamped to the matrix), physical chunk l % CPR,
    // i.e. logical chunk (l % CPR) ^ key(row).  M-/N-contiguous operand:
    // k-row (64 q' + l) / CPK of the operand's part (q' counted from the
    // part's first group), slot (l % CPK), i.e. logical chunk mn_slot of
    // it, at a column clamped as described above.  Byte offsets are
    // relative to the tile origin at the stage's first k.
    uint32_t voff[LPW];
    bool from_a[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = wave * LPW + i;
        from_a[i] = q < A_GROUPS;                     // per group, hence wave-uniform
        const bool mn = from_a[i] ? AT : BT;
        if (mn) {
            const int cpk = from_a[i] ? A_CPK : B_CPK;
            const int qp = from_a[i] ? q : q - A_GROUPS;
            const int k = (64 * qp + lane) / cpk;
            const int c = mn_slot(lane % cpk, k);
            const int64_t ext = from_a[i] ? a_ext : b_ext;
            const int64_t cmax = 8 * ((ext - 1) / 8);    // last chunk starting inside
            const int64_t col = 8 * c < cmax ? 8 * c : cmax;
            voff[i] = (uint32_t)((k * (from_a[i] ? lda : ldb) + col) * 2);
        } else {
            const int srow = q * RPI + lane / CPR;                     // stage row
            const int c = (lane % CPR) ^ swizzle_key<CPR>(srow);       // logical chunk
            int64_t r = from_a[i] ? srow : srow - BM;     // row inside the A / B tile
            const int64_t lim = from_a[i] ? a_ext : b_ext;
            r = r < lim ? r : lim - 1;
            voff[i] = (uint32_t)((r * (from_a[i] ? lda : ldb) + c * 8) * 2);
        }
    }

    // K position of virtual tile v: a register-loaded tile (if any) comes
    // first: the partial last K tile, or, where an M- or N-contiguous
    // operand's edge cuts a chunk and this K range ends at K, the last full
    // K tile.
    const int64_t klen = ke > kb ? ke - kb : 0;
    const bool cut_edge = ke == g.K && ((AT && a_ext % 8 != 0) || (BT && b_ext % 8 != 0));
    const bool tail = (klen % MBK) != 0 || (cut_edge && klen > 0);
    const int64_t nfull = (klen % MBK) != 0 ? klen / MBK : (tail ? klen / MBK - 1 : klen / MBK);
    const int64_t ntiles = nfull + (tail ? 1 : 0);
    auto tile_k0 = [&](int64_t v) -> int64_t {
        if (tail)
            return v == 0 ? kb + nfull * MBK : kb + (v - 1) * MBK;
        return kb + v * MBK;
    };

    // Source of DMA group i at K position k0: the tile origin advanced by
    // k0 along K (one element per k for a K-contiguous operand, one leading
    // dimension for an M- or N-contiguous one).  One expression for both
    // operands (a pointer and a step chosen by the group): with a separate
    // expression per operand the compiler branches around every DMA
    // instruction of a mixed-layout kernel and its K loop loses the
    // interleaved schedule.
    const int64_t a_step = AT ? lda : 1, b_step = BT ? ldb : 1;
    auto group_base = [&](int i, int64_t k0) -> const uint16_t * {
        return (from_a[i] ? A_tile : B_tile) + k0 * (from_a[i] ? a_step : b_step);
    };

    // DMA instruction i (of LPW) of full tile v into its stage.
    auto issue_dma_one = [&](int64_t v, int i) {
        const int64_t k0 = tile_k0(v);
        const uint32_t dst = lds_base + (uint32_t)((v % kStages) * STAGE_SLOTS * 16) +
                             (uint32_t)((wave * LPW + i) * 1024);
#ifdef DG_LOAD_POLICY
        dma_16_policy(from_a[i], uniform_ptr(group_base(i, k0)), voff[i], dst);
#else
        dma_16(uniform_ptr(group_base(i, k0)), voff[i], dst);
#endif
    };
    auto issue_dma = [&](int64_t v) {
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            issue_dma_one(v, i);
    };

    // The register-loaded tile: same slots as the DMA, with the K mask (and
    // the M / N mask on an M- or N-contiguous operand).  Every chunk's load
    // is issued before the first LDS write, so the wave waits for memory
    // once, not once per chunk.  With ke a multiple of 8 (uniform) no chunk
    // straddles it: a K-contiguous chunk is then one 16-byte load from a
    // clamped (valid) position, zeroed past ke, with no branch.
    auto tail_chunk = [&](int i, int64_t k0, bool k_whole) -> uint4 {
        const int q = wave * LPW + i;
        const bool mn = from_a[i] ? AT : BT;
        if (mn) {
            const int cpk = from_a[i] ? A_CPK : B_CPK;
            const int qp = from_a[i] ? q : q - A_GROUPS;
            const int k = (64 * qp + lane) / cpk;
            const int c = mn_slot(lane % cpk, k);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (k0 + k < ke) {
                const int64_t ld = from_a[i] ? lda : ldb;
                const uint16_t *row = (from_a[i] ? A_tile : B_tile) + (k0 + k) * ld;
                val = load_chunk_cols(row, 8 * c, from_a[i] ? a_ext : b_ext);
            }
            return val;
        }
        const int srow = q * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swizzle_key<CPR>(srow);
        const uint16_t *rowp = (const uint16_t *)((const char *)(from_a[i] ? A_tile : B_tile) +
                                                  voff[i]) - c * 8;
        const int64_t kf = k0 + c * 8;
        if (k_whole) {
            const uint4 x = *(const uint4 *)(rowp + (kf < ke ? kf : ke - 8));
            return kf < ke ? x : make_uint4(0u, 0u, 0u, 0u);
        }
        return load_chunk_tail(rowp, kf, ke);
    };
    auto load_tail = [&](int64_t v) {
        const int64_t k0 = tile_k0(v);
        uint4 vals[LPW];
        if ((ke & 7) == 0) {
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                vals[i] = tail_chunk(i, k0, true);
        } else {
#pragma unroll
            for (int i = 0; i < LPW; ++i)
                vals[i] = tail_chunk(i, k0, false);
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i)
            lds[(v % kStages) * STAGE_SLOTS + (wave * LPW + i) * 64 + lane] = vals[i];
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                acc[i][j][v] = 0.0f;

    const int frag_row = lane % MS;       // row of A / column of B this lane feeds
    const int frag_grp = lane / MS;       // which 8 of the KD k of one MFMA step
    const int swz = swizzle_key<CPR>(frag_row);   // key of every fragment row (period 16)
    // Transposing reads: lane 16g + 4r + q addresses k-row 8 (g / 2) + r of
    // a k-step and columns 16 (g mod 2) + 4q .. + 3 of a fragment (see
    // tr_fragment).  Byte offset of that piece inside an M-/N-contiguous
    // part, k-step 0, first read, for the wave's fragment i (A) or j (B).
    // With 16 x 16 blocks lane 16g + 4r + q addresses k-row 8g + r and
    // columns 4q .. + 3 of the 16-column fragment, so lane 16g + i receives
    // k-rows 8g .. 8g + 3 (and 8g + 4 .. 8g + 7 from the second read) of
    // column i.
    const int tr_g = lane >> 4, tr_r = (lane >> 2) & 3, tr_q = lane & 3;
    const int tr_krow = MS == 32 ? 8 * (tr_g >> 1) + tr_r : 8 * tr_g + tr_r;
    // chunk inside the fragment's columns
    const int tr_chunk = MS == 32 ? 2 * (tr_g & 1) + (tr_q >> 1) : tr_q >> 1;
    uint32_t a_tr[AT ? FM : 1], b_tr[BT ? FN : 1];
    if constexpr (AT) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            a_tr[i] = (uint32_t)(tr_krow * BM * 2 +
                                 16 * mn_slot((wm * TM + MS * i) / 8 + tr_chunk, tr_krow) +
                                 8 * (tr_q & 1));
    }
    if constexpr (BT) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            b_tr[j] = (uint32_t)(tr_krow * BN * 2 +
                                 16 * mn_slot((wn * TN + MS * j) / 8 + tr_chunk, tr_krow) +
                                 8 * (tr_q & 1));
    }

    auto mfma_step = [&](const frag_t *af, const frag_t *bf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mfma_block(af[i], bf[j], acc[i][j]);
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
    // a_off / b_off: LDS byte offsets of A's and B's part of the stage;
    // issue(d) runs after the MFMA of slot d (DMA of later tiles).
    auto stage_body = [&](uint32_t a_off, uint32_t b_off, auto &&issue) {
        const uint4 *as = lds + a_off / 16 + (wm * TM + frag_row) * CPR;
        const uint4 *bs = lds + b_off / 16 + (wn * TN + frag_row) * CPR;
        const uint32_t a_addr = lds_base + a_off, b_addr = lds_base + b_off;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1, prev = cur ^ 1;
            const int c = (ks * CPS + frag_grp) ^ swz;
#pragma unroll
            for (int n = 0; n < FM * FN; ++n) {
                if (n < FM) {
                    if constexpr (AT)
                        fa[cur][n] = tr_fragment<frag_t, BM * 2>(a_addr + a_tr[n] +
                                                                  KD * ks * BM * 2);
                    else
                        fa[cur][n] = __builtin_bit_cast(frag_t, as[n * MS * CPR + c]);
                } else if (n < FM + FN) {
                    if constexpr (BT)
                        fb[cur][n - FM] = tr_fragment<frag_t, BN * 2>(b_addr + b_tr[n - FM] +
                                                                       KD * ks * BN * 2);
                    else
                        fb[cur][n - FM] = __builtin_bit_cast(frag_t, bs[(n - FM) * MS * CPR + c]);
                }
                const int i = n / FN, j = n % FN;
                acc[i][j] = mfma_block(fa[prev][i], fb[prev][j], acc[i][j]);
                issue(ks * FM * FN + n);
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
        auto no_dma = [](int) {};
        // prologue: tiles 0 .. D-1; with a register-loaded tile 0 the DMA of
        // tiles 1 .. D-1 goes first, so that both are in flight together
        if (tail) {
            for (int64_t v = 1; v < D && v < ntiles; ++v)
                issue_dma(v);
            load_tail(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the register-path LDS writes
        } else {
            for (int64_t v = 0; v < D && v < ntiles; ++v)
                issue_dma(v);
        }
        auto stage_off = [](int64_t v) -> uint32_t {
            return (uint32_t)((v % kStages) * STAGE_SLOTS * 16);
        };
        constexpr uint32_t B_OFF = (uint32_t)BM * MBK * 2;   // B's rows follow A's
        int64_t v = 0;
        // steady state: D-1 later tiles stay in flight while tile v is used
        for (; v + D < ntiles; ++v) {
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm((D - 1) * LPW));
            barrier();
            stage_body(stage_off(v), stage_off(v) + B_OFF, [&](int d) {
                if (d % MFMA_PER_DMA == MFMA_PER_DMA - 1 && d / MFMA_PER_DMA < LPW)
                    issue_dma_one(v + D, d / MFMA_PER_DMA);
            });
        }
        // drain
        for (; v < ntiles; ++v) {
            __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
            barrier();
            stage_body(stage_off(v), stage_off(v) + B_OFF, no_dma);
        }
        mfma_step(fa[1], fb[1]);   // last k-step of the last stage
        __builtin_amdgcn_s_waitcnt(vm_lgkm0_imm(0));
        barrier();
    }

    // the epilogue keeps within the kernel's register budget
    constexpr int REGS = 512 / mfma16_per_cu(BM, BN, kStages, MBK);
    if constexpr (MS == 32) {
        if (part)
            tile_epilogue_rows<BM, BN, WM, WN, true, DT_F32, REGS, false>(
                g, (char *)part, BN, BM, BN, n0, (float *)lds, acc);
        else
            tile_epilogue<BM, BN, WM, WN, REGS>(g, tc, (float *)lds, m0, n0, acc);
    } else {
        const Acc16View<FM, FN> view{acc};
        if (part)
            tile_epilogue_rows<BM, BN, WM, WN, true, DT_F32, REGS, false>(
                g, (char *)part, BN, BM, BN, n0, (float *)lds, view);
        else
            tile_epilogue<BM, BN, WM, WN, REGS>(g, tc, (float *)lds, m0, n0, view);
    }
}

// Data-parallel launches give each program one tile (or split-K slice).
// Stream-K launches give programs [0, dp_tiles) one whole tile each and the
// others one K slice of a tail tile, written as a raw fp32 partial that the
// fix-up kernel adds up.
template <int T, int BM, int BN, int WM, int WN, int kStages, int MBK, bool AT, bool BT, int MS>
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
        const uint32_t tt = (uint32_t)sk.tail_tiles;   // 32-bit, as the grid
        const int64_t slice = (uint32_t)i / tt, r = (uint32_t)i % tt;
        tc = decode_tile(sk.dp_tiles + r, g.sched);
        kb = slice * sk.k_per_split;
        ke = kb + sk.k_per_split < g.K ? kb + sk.k_per_split : g.K;
        part = g.sk_parts + (r * sk.tail_splits + slice) * (int64_t)(BM * BN);
    }
    mfma16_tile<T, BM, BN, WM, WN, kStages, MBK, AT, BT, MS>(g, tc, kb, ke, part, lds);
}

// One kernel name per element type, so that traces tell them apart.  AT /
// BT: A stored M-contiguous (column-major) / B stored N-contiguous
// (row-major).
template <int BM, int BN, int WM, int WN, int kStages, int MBK, bool AT, bool BT, int MS>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(mfma16_per_cu(BM, BN, kStages, MBK))))
void gemm_mfma_bf16_kernel(GemmArgs g)
{
    if (g.sliver_blocks && (int64_t)blockIdx.x >= g.main_programs) {
        // 32-bit (the grid is): a 64-bit division here costs the whole
        // kernel scalar registers
        const uint32_t i = blockIdx.x - (uint32_t)g.main_programs;
        const uint32_t nb = (uint32_t)g.sliver_blocks;
        sliver_block<DT_BF16, 1>(g, g.sliver_n0, 1, i % nb, i / nb);
        return;
    }
    extern __shared__ uint4 lds[];
    mfma16_program<DT_BF16, BM, BN, WM, WN, kStages, MBK, AT, BT, MS>(g, lds);
}

template <int BM, int BN, int WM, int WN, int kStages, int MBK, bool AT, bool BT, int MS>
__global__ __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(mfma16_per_cu(BM, BN, kStages, MBK))))
void gemm_mfma_f16_kernel(GemmArgs g)
{
    if (g.sliver_blocks && (int64_t)blockIdx.x >= g.main_programs) {
        // 32-bit (the grid is): a 64-bit division here costs the whole
        // kernel scalar registers
        const uint32_t i = blockIdx.x - (uint32_t)g.main_programs;
        const uint32_t nb = (uint32_t)g.sliver_blocks;
        sliver_block<DT_F16, 1>(g, g.sliver_n0, 1, i % nb, i / nb);
        return;
    }
    extern __shared__ uint4 lds[];
    mfma16_program<DT_F16, BM, BN, WM, WN, kStages, MBK, AT, BT, MS>(g, lds);
}

template <int T, int BM, int BN, int WM, int WN, int NS, int BK, bool AT, bool BT, int MS = 32>
hipError_t launch_layout(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const size_t lds_bytes = (size_t)mfma16_lds_bytes(BM, BN, NS, BK, MS);
    static_assert(mfma16_per_cu(BM, BN, NS, BK) ==
                      160 * 1024 / mfma16_lds_bytes(BM, BN, NS, BK, MS) ||
                      mfma16_per_cu(BM, BN, NS, BK) < 160 * 1024 / mfma16_lds_bytes(BM, BN, NS, BK, MS),
                  "the 16 x 16 epilogue's staging keeps the tile's occupancy");
    static_assert(64 * WM * WN == kSliverThreads, "sliver workgroups share the kernel's block");
    const int64_t programs = p.programs + g.sliver_blocks * g.sched.batch;
    const dim3 grid((unsigned)programs), block(64 * WM * WN);
    if constexpr (T == DT_F16)
        hipLaunchKernelGGL((gemm_mfma_f16_kernel<BM, BN, WM, WN, NS, BK, AT, BT, MS>), grid, block,
                           lds_bytes, stream, g);
    else
        hipLaunchKernelGGL((gemm_mfma_bf16_kernel<BM, BN, WM, WN, NS, BK, AT, BT, MS>), grid, block,
                           lds_bytes, stream, g);
    return hipGetLastError();
}

// K-contiguous A and B (A row-major, B column-major) on any tile; the
// other three layouts on the tiles of the automatic choice (the 256 x 256
// and 128 x 128 tiles), which the planner restricts them to.
template <int T, int BM, int BN, int WM, int WN, int NS, int BK, int MS = 32>
hipError_t launch_one(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    return launch_layout<T, BM, BN, WM, WN, NS, BK, false, false, MS>(g, p, stream);
}

template <int T, int BM, int BN, int WM, int WN, int NS, int BK>
hipError_t launch_any_layout(const GemmArgs &g, const Plan &p, hipStream_t stream)
{
    const bool at = g.a_col != 0, bt = g.b_col == 0;
    if (at && bt)
        return launch_layout<T, BM, BN, WM, WN, NS, BK, true, true>(g, p, stream);
    if (at)
        return launch_layout<T, BM, BN, WM, WN, NS, BK, true, false>(g, p, stream);
    if (bt)
        return launch_layout<T, BM, BN, WM, WN, NS, BK, false, true>(g, p, stream);
    return launch_layout<T, BM, BN, WM, WN, NS, BK, false, false>(g, p, stream);
}

} // namespace

// Launchers of the instantiation files: K-contiguous bf16 and fp16 tiles
// (variants 0-4 and 5-9 of each), and the M- or
// N-contiguous layouts on the 256 x 256 (variant 5) and 128 x 128 (variant
// 1) tiles of either type.
hipError_t launch_mfma16_bf16_a(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma16_bf16_b(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma16_f16_a(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma16_f16_b(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma16_mn256(const GemmArgs &g, const Plan &p, hipStream_t stream);
hipError_t launch_mfma16_mn128(const GemmArgs &g, const Plan &p, hipStream_t stream);

} // namespace dg
