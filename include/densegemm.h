/*
 * densegemm.h -- C ABI of an MI355X (gfx950) dense GEMM library.
 *
 * Operation (one call, optionally batched):
 *
 *     C[b] = act( alpha * A[b] . B[b] + beta * C[b] + bias )      b < batch
 *
 * with A[b] an M x K matrix, B[b] a K x N matrix, C[b] an M x N matrix, the
 * product accumulated in fp32 and rounded to C's dtype only after the whole
 * K loop.  The problem statement is the one of "La GEMM, de zero a cuBLAS"
 * section 2.1; the list of inputs (M, N, K, dtype, per-operand layout,
 * output dtype, epilogue with alpha / bias / activation / accumulation into
 * an existing C, batched or broadcast operands) follows "Skill: Write a
 * Triton GEMM Kernel", section "Inputs the agent should gather first"; the
 * rule that every stride is an argument and that a broadcast operand has
 * batch stride 0 follows the same page's "Kernel design rules" and
 * "Correctness requirements".
 *
 * Conventions
 *   - Plain C99.  Every pointer argument named A, B, C, bias or workspace is
 *     a DEVICE pointer; the descriptor and text buffers are HOST pointers.
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     or frees device memory and keeps no pointer after a call returns,
 *     apart from the work it has enqueued; the caller keeps the buffers alive
 *     until that work has completed on `stream`.  The descriptor is read only
 *     during the call.
 *   - Asynchrony: work is enqueued on `stream` (NULL = the null stream) and
 *     the library never synchronises.  Results of one call are ordered
 *     before later work on the same stream.
 *   - Errors: return codes only.  Every argument is validated on the host
 *     before anything is enqueued, so any status other than DG_SUCCESS and
 *     DG_ERROR_LAUNCH means nothing was enqueued.  The only mutable global
 *     state is the per-device address of dg_gemm_noalloc's scratch array,
 *     looked up once under a lock; calls are thread-safe and reentrant
 *     (dg_gemm_noalloc calls that overlap on one GPU share its scratch; see
 *     there).
 *   - Determinism: results are bitwise reproducible run to run for a given
 *     descriptor, including split-K (partials are reduced in a fixed order,
 *     never with atomics).
 */
#ifndef DENSEGEMM_H
#define DENSEGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_VERSION 10000 /* 1.0.0 */

/* Status codes. */
typedef enum {
    DG_SUCCESS = 0,
    DG_ERROR_INVALID_VALUE = 1,          /* malformed descriptor or pointers */
    DG_ERROR_NOT_SUPPORTED = 2,          /* valid, but not a supported combination */
    DG_ERROR_INSUFFICIENT_WORKSPACE = 3, /* forced split-K without enough workspace */
    DG_ERROR_LAUNCH = 4                  /* the runtime refused a kernel launch */
} dg_status;

/* Element types.  DG_BF16 is bfloat16: the top 16 bits of an IEEE fp32.
 * DG_F16 is IEEE 754 binary16 (5 exponent bits, 10 fraction bits; largest
 * finite value 65504).  Inputs in fp16 are the dtype of the pages' own
 * correctness check ("Skill: Write a Triton GEMM Kernel", Inputs the agent
 * should gather first, and the allclose check of "GEMM Kernel
 * Optimization", Verification). */
typedef enum { DG_F32 = 0, DG_BF16 = 1, DG_F16 = 2 } dg_dtype;

/* Storage order of one operand.  Row-major X (R x C) with leading dimension
 * ld holds X[r][c] at element r*ld + c; column-major holds it at c*ld + r. */
typedef enum { DG_ROW_MAJOR = 0, DG_COL_MAJOR = 1 } dg_order;

/* Epilogue activation, applied to alpha*acc + beta*C + bias.
 * GELU_ERF is x * Phi(x) with Phi the standard normal CDF;
 * GELU_TANH replaces Phi(x) by (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))/2. */
typedef enum { DG_ACT_NONE = 0, DG_ACT_GELU_ERF = 1, DG_ACT_GELU_TANH = 2 } dg_act;

/* Kernel family selection (benchmarking and ablation; 0 lets the library
 * choose).  GENERIC is the plain LDS-tiled kernel that serves every
 * layout, alignment and dtype.  For fp32 the automatic choice is the
 * matrix-core kernel (MFMA_F32) when the operands are 16-byte aligned with
 * leading dimensions and batch strides multiple of 4; VALU_F32 (the
 * register-tiled vector-FMA kernel) takes the same operands and is used
 * only when asked for.  bf16 and fp16 inputs go to their matrix-core kernel
 * (MFMA_BF16, MFMA_F16) in any order of A and B, both 16-byte aligned with
 * leading dimensions and batch strides multiple of 8 (a column-major A or
 * row-major B is transposed on its way from LDS to the matrix cores).
 * Forcing a family whose requirements the operands do not meet returns
 * DG_ERROR_NOT_SUPPORTED. */
typedef enum {
    DG_ALGO_AUTO = 0,
    DG_ALGO_GENERIC = 1,
    DG_ALGO_VALU_F32 = 2,  /* register-tiled fp32 outer-product kernel */
    DG_ALGO_MFMA_BF16 = 3, /* bf16 matrix-core kernel */
    DG_ALGO_MFMA_F32 = 4,  /* fp32 matrix-core kernel */
    DG_ALGO_MFMA_F16 = 5   /* fp16 matrix-core kernel (the bf16 kernel's twin) */
} dg_algo;

/* Work distribution over the compute units (benchmarking and ablation; 0
 * lets the library choose).  DATA_PARALLEL gives every output tile (and
 * split-K slice) to one workgroup.  STREAM_K splits work along K to keep
 * the last wave busy ("La GEMM, de zero a cuBLAS", section 2.10, on
 * Stream-K and wave quantisation): the tiles of the full waves stay
 * data-parallel, and the K range of each remaining (tail) tile is cut into
 * slices, one workgroup each, enough to fill one more wave; a second, small
 * kernel adds each tail tile's fp32 partials in slice order (fixed order, no
 * atomics) and applies the epilogue; with STREAM_K, split_k = S > 1 cuts
 * each tail tile's K range into slices of ceil(K / S) rounded up to whole K
 * steps (so possibly fewer than S slices) instead of a split-K count.  STREAM_K applies to the bf16 and fp16 matrix-core
 * kernels with batch == 1 and needs workspace
 * (see dg_gemm_workspace_size); otherwise DG_ERROR_NOT_SUPPORTED.  The
 * automatic choice uses it only for those kernels, when there is at least
 * one full wave of tiles, the last wave would be less than 85 % full,
 * K >= 2048 and the caller passes enough workspace, or where the
 * offline-tuned plan table names it for the exact shape.
 *
 * With schedule, algo and split_k all left to the library, an output whose
 * N ends 1 to 8 columns past a whole number of tile columns (for the tile
 * the plan chose), with row-major A whose rows are 16-byte aligned, at
 * least one full-width tile per compute unit, and one wave of tiles fewer
 * without the last tile column, is computed in two launches
 * on the stream: the tiled plan over the full tile columns, then a small
 * kernel over the last columns (one wavefront per row of A, each output a
 * K-long fp32 dot product, the same epilogue).  A tuned stream-K plan with
 * a tail wave keeps the whole grid instead.  Results agree with the single
 * tiled plan within the dtype's tolerance (bit for bit when every product
 * and partial sum is exact in fp32). */
typedef enum {
    DG_SCHED_AUTO = 0,
    DG_SCHED_DATA_PARALLEL = 1,
    DG_SCHED_STREAM_K = 2
} dg_schedule;

/*
 * Problem descriptor.  All integer fields are in ELEMENTS, not bytes.
 *
 *   struct_size     must be sizeof(dg_gemm_desc) (ABI versioning).
 *   M, N, K         >= 0.  M == 0 or N == 0 is a successful no-op; K == 0
 *                   gives C = act(beta*C + bias).
 *   batch           >= 0; 0 is a no-op.
 *   a_type, b_type  input types; c_type output type.  Supported
 *                   (a, b, c): (F32, F32, F32), and for 16-bit inputs
 *                   (X, X, c) with X = BF16 or F16 and c = F32, BF16 or
 *                   F16.  Accumulation is always fp32; a 16-bit output is
 *                   rounded to nearest, ties to even (fp16 beyond 65504
 *                   rounds to infinity).
 *   a_order ...     storage order of A (M x K), B (K x N), C (M x N).
 *   lda, ldb, ldc   leading dimensions, each >= max(1, length of the
 *                   contiguous dimension) (e.g. row-major A: lda >= K).
 *   stride_a/b/c    batch strides, >= 0.  stride_a == 0 (or stride_b == 0)
 *                   broadcasts one A (B) to every batch entry.
 *                   stride_c must not make two C matrices overlap.
 *   alpha, beta     host scalars.  beta == 0: C is not read (NaN in C does
 *                   not propagate).  alpha == 0: A and B are not read.
 *   bias, bias_type optional DEVICE vector of N elements (F32, BF16 or F16),
 *                   added to every row; NULL for none.
 *   act             activation, see dg_act.
 *   split_k         0: the library decides (it only splits K when the
 *                   caller passes enough workspace); 1: never split;
 *                   S > 1: split K into S slices (needs workspace); with
 *                   schedule STREAM_K, the K slices of each tail tile.
 *   group_m         output-tile group height of the swizzled tile order; 0
 *                   picks the default (4, measured best with the XCD
 *                   remap).  1 gives plain row-major order.
 *   algo            dg_algo; 0 = automatic choice.
 *   xcd_remap       1 (default when 0) spreads consecutive tile groups over
 *                   the chip's 8 XCDs so each XCD's L2 sees a contiguous
 *                   part of the swizzled order; -1 disables it.
 *   schedule        dg_schedule; 0 = automatic choice.
 */
typedef struct dg_gemm_desc {
    uint32_t struct_size;
    int32_t a_type, b_type, c_type;   /* dg_dtype */
    int64_t M, N, K, batch;
    int32_t a_order, b_order, c_order; /* dg_order */
    int32_t bias_type;                 /* dg_dtype */
    int64_t lda, ldb, ldc;
    int64_t stride_a, stride_b, stride_c;
    float alpha, beta;
    const void *bias;
    int32_t act;       /* dg_act */
    int32_t split_k;
    int32_t group_m;
    int32_t algo;      /* dg_algo */
    int32_t xcd_remap;
    int32_t schedule;  /* dg_schedule */
} dg_gemm_desc;

/* Library version, DG_VERSION of the build. */
int dg_version(void);

/* Static text for a status code; never NULL. */
const char *dg_status_string(dg_status s);

/* Device bytes of workspace that dg_gemm would use for `d` (0 when the
 * chosen plan needs none).  The workspace holds fp32 partial sums: of
 * every K slice of a split-K plan, reduced in a separate pass ("Skill:
 * Write a Triton GEMM Kernel", Kernel design rules, on split-K), or of the
 * tail tiles' K slices of a stream-K plan.  With split_k == 0 and schedule == 0 this is the
 * size that lets the library pick split-K or Stream-K where they pay.  Returns INVALID_VALUE /
 * NOT_SUPPORTED for descriptors dg_gemm would reject. */
dg_status dg_gemm_workspace_size(const dg_gemm_desc *d, size_t *bytes);

/* Enqueue C = act(alpha*A.B + beta*C + bias) on `stream`.
 *   A, B, C    device pointers to the matrices (C is read when beta != 0
 *              and written); they must be aligned to their element size.
 *              C must not overlap A, B or bias.  A and B may be NULL when
 *              alpha == 0 or K == 0.
 *   workspace  device scratch of workspace_bytes (may be NULL / 0),
 *              16-byte aligned.  The library writes it; its content before
 *              and after is unspecified.  It must not be used by other work
 *              until this call's work has completed on `stream`.
 *   stream     a hipStream_t (passed as void*), NULL for the null stream.
 * Returns DG_SUCCESS once the work is enqueued. */
dg_status dg_gemm(const dg_gemm_desc *d, const void *A, const void *B, void *C,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Size in bytes of the per-GPU scratch array of dg_gemm_noalloc. */
#define DG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* dg_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same operation, arguments (minus the workspace), validation, plans and
 * results as dg_gemm given DG_NOALLOC_SCRATCH_BYTES of workspace, except
 * that split-K and stream-K partials go to a scratch array of that size
 * that is part of the library's device code: each GPU the library runs on
 * holds one copy from the library's load until the process ends, and no
 * call allocates or frees anything (no hipMalloc / hipFree, no allocating
 * library routine).  The first call on a device looks up that device's copy
 * (hipGetSymbolAddress, with the device current); later calls reuse it.
 *   - The automatic choice never plans more than DG_NOALLOC_SCRATCH_BYTES
 *     of workspace.  A forced split_k or STREAM_K schedule whose workspace
 *     (see dg_gemm_workspace_size) exceeds it returns
 *     DG_ERROR_INSUFFICIENT_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's partials; nothing in it needs to start at zero.  Calls whose
 *     work overlaps in time on one GPU (other streams, other host threads)
 *     race on it: order them on one stream or serialise them.
 *   - DG_ERROR_LAUNCH also covers a failed device or symbol lookup. */
dg_status dg_gemm_noalloc(const dg_gemm_desc *d, const void *A, const void *B, void *C,
                          void *stream);

/* Write a one-line, NUL-terminated description of the plan dg_gemm would
 * run for `d` (kernel, tile, split, grid, workspace) into buf[len].  Pass
 * workspace_bytes as dg_gemm would receive it (it decides split-K when
 * split_k == 0).  "sliver=n" (n > 0) marks the two-launch split above:
 * the rest of the line then describes the tiled plan over the first N - n
 * columns.  "tuned=1" marks a plan taken from the library's
 * offline-tuned table: for the exact (kernel family, M, N, K, batch) of a
 * shape swept on an MI355X, the tile and schedule that measured fastest
 * replace the heuristic choice ("GEMM Kernel Optimization", Autotune
 * Configs; "Skill: Write a Triton GEMM Kernel", Required reasoning process
 * step 7; with the benchmarking done once, offline). */
dg_status dg_gemm_describe(const dg_gemm_desc *d, size_t workspace_bytes, char *buf,
                           size_t len);

/* Host-side evaluation of the tile scheduler, for checking its bijection:
 * for every program id p < P = batch * S * ceil(M/bm) * ceil(N/bn) writes
 * out[4p .. 4p+3] = (batch index, split index, tile row, tile column) that
 * a kernel launched with that grid gives program p.  `out` is a HOST array
 * of 4*P int32.  Uses exactly the code the kernels use, which is 32-bit:
 * P above 2^31 - 1 (more programs than any launch can have) returns
 * DG_ERROR_NOT_SUPPORTED. */
dg_status dg_schedule_map(int64_t M, int64_t N, int64_t batch, int32_t split_k, int32_t bm,
                          int32_t bn, int32_t group_m, int32_t xcd_remap, int32_t *out,
                          int64_t out_len);

#ifdef __cplusplus
}
#endif
#endif /* DENSEGEMM_H */
