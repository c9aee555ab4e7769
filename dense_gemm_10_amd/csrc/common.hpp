// Device-side building blocks shared by the GEMM kernels: the kernel
// argument block, typed element access with per-operand order / leading
// dimension / batch stride, bf16 conversion and the fused epilogue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scheduler.hpp"

namespace dg {

// Everything a kernel needs, passed by value (one kernarg block).
struct GemmArgs {
    const void *A;
    const void *B;
    void *C;
    const void *bias;
    float *ws;                 // split-K partials, [split][batch][M][N] fp32
    int64_t M, N, K;
    int64_t lda, ldb, ldc;
    int64_t sa, sb, sc;        // batch strides (elements)
    int64_t k_per_split;       // K range of one split (multiple of the kernel's BK)
    float alpha, beta;
    int32_t a_col, b_col, c_col;   // 1 = column-major
    int32_t c_bf16;                // output dtype: 1 = bf16, 0 = fp32
    int32_t bias_bf16;
    int32_t act;                   // dg_act
    int32_t write_partial;         // 1: store raw fp32 partials to ws, no epilogue
    int32_t ab_bf16;               // input dtype of A and B: 1 = bf16, 0 = fp32
    int32_t out_vec16;             // 1: the output (C, or ws when write_partial) is
                                   // row-major and every row of every batch entry
                                   // starts on a 16-byte boundary
    SchedArgs sched;
};

enum { ACT_NONE = 0, ACT_GELU_ERF = 1, ACT_GELU_TANH = 2 };

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest, ties to even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// ---- typed loads -------------------------------------------------------------
__device__ __forceinline__ int64_t elem_offset(int32_t col_major, int64_t ld, int64_t r,
                                               int64_t c)
{
    return col_major ? c * ld + r : r * ld + c;
}

__device__ __forceinline__ float load_as_f32(const void *base, int32_t is_bf16, int64_t idx)
{
    return is_bf16 ? bf16_to_f32(((const uint16_t *)base)[idx]) : ((const float *)base)[idx];
}

// ---- activation ------------------------------------------------------------
__device__ __forceinline__ float activate(float x, int32_t act)
{
    if (act == ACT_GELU_ERF)
        return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));   // x * Phi(x)
    if (act == ACT_GELU_TANH) {
        const float s = 0.79788456080286536f;                          // sqrt(2/pi)
        return 0.5f * x * (1.0f + tanhf(s * (x + 0.044715f * x * x * x)));
    }
    return x;
}

// ---- epilogue --------------------------------------------------------------
// Applied once per output element after the whole K loop ("Skill: Write a
// Triton GEMM Kernel", Required reasoning process step 6, and the alpha /
// beta failure mode): v = act(alpha*acc + beta*C + bias[n]), then the cast
// to C's dtype.  beta == 0 never reads C.
__device__ __forceinline__ float epilogue_value(const GemmArgs &g, int64_t b, int64_t m,
                                                int64_t n, float acc)
{
    float v = g.alpha * acc;
    if (g.beta != 0.0f) {
        int64_t ci = b * g.sc + elem_offset(g.c_col, g.ldc, m, n);
        v = fmaf(g.beta, load_as_f32(g.C, g.c_bf16, ci), v);
    }
    if (g.bias)
        v += load_as_f32(g.bias, g.bias_bf16, n);
    return activate(v, g.act);
}

__device__ __forceinline__ void store_c(const GemmArgs &g, int64_t b, int64_t m, int64_t n,
                                        float v)
{
    int64_t ci = b * g.sc + elem_offset(g.c_col, g.ldc, m, n);
    if (g.c_bf16)
        ((uint16_t *)g.C)[ci] = f32_to_bf16(v);
    else
        ((float *)g.C)[ci] = v;
}

// Final value or split-K partial for output (b, m, n) of split s.
__device__ __forceinline__ void write_result(const GemmArgs &g, int64_t b, int32_t s,
                                             int64_t m, int64_t n, float acc)
{
    if (g.write_partial) {
        int64_t wi = (((int64_t)s * g.sched.batch + b) * g.M + m) * g.N + n;
        g.ws[wi] = acc;
    } else {
        store_c(g, b, m, n, epilogue_value(g, b, m, n, acc));
    }
}

// K range [k_begin, k_end) handled by split s.
__device__ __forceinline__ void split_range(const GemmArgs &g, int32_t s, int64_t &k_begin,
                                            int64_t &k_end)
{
    k_begin = (int64_t)s * g.k_per_split;
    k_end = k_begin + g.k_per_split;
    if (k_end > g.K)
        k_end = g.K;
    if (k_begin > g.K)
        k_begin = g.K;
}

} // namespace dg
