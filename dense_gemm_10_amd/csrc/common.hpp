// Device-side building blocks shared by the GEMM kernels: the kernel
// argument block, typed element access with per-operand order / leading
// dimension / batch stride, bf16 / fp16 conversion and the fused epilogue.
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
    int32_t c_type;                // output dtype (DT_*)
    int32_t bias_type;             // bias dtype (DT_*)
    int32_t act;                   // dg_act
    int32_t write_partial;         // 1: store raw fp32 partials to ws, no epilogue
    int32_t ab_type;               // dtype of A and B (DT_*)
    SchedArgs sched;
    StreamK sk;                    // sk.tail_tiles == 0: data-parallel launch
    float *sk_parts;               // stream-K partials, [tail tile][slice][BM * BN] fp32
    // One sliver column (output column sliver_n0) run by a tiled kernel as
    // extra workgroups after its main_programs tile programs, with
    // sliver_blocks (per batch entry) of rows each; 0 sliver_blocks: none.
    int64_t sliver_n0;
    int64_t main_programs;
    int64_t sliver_blocks;
};

enum { ACT_NONE = 0, ACT_GELU_ERF = 1, ACT_GELU_TANH = 2 };
// element types, numbered as dg_dtype
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// ---- 16-bit floats <-> fp32 -----------------------------------------------
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

// IEEE binary16: exact widening; narrowing rounds to nearest, ties to even
// (hardware conversion), beyond the largest finite value to infinity.
__device__ __forceinline__ float f16_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16(float x)
{
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// One 16-bit element of type T (DT_BF16 or DT_F16) <-> fp32.
template <int T>
__device__ __forceinline__ float half_to_f32(uint16_t h)
{
    return T == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h);
}

template <int T>
__device__ __forceinline__ uint16_t f32_to_half(float x)
{
    return T == DT_F16 ? f32_to_f16(x) : f32_to_bf16(x);
}

// ---- typed loads -------------------------------------------------------------
__device__ __forceinline__ int64_t elem_offset(int32_t col_major, int64_t ld, int64_t r,
                                               int64_t c)
{
    return col_major ? c * ld + r : r * ld + c;
}

__device__ __forceinline__ float load_as_f32(const void *base, int32_t type, int64_t idx)
{
    if (type == DT_F32)
        return ((const float *)base)[idx];
    const uint16_t h = ((const uint16_t *)base)[idx];
    return type == DT_F16 ? f16_to_f32(h) : bf16_to_f32(h);
}

// ---- activation ------------------------------------------------------------
// GELU with the exact normal CDF, x * Phi(x), where Phi(x) = 1 - h for
// x >= 0 and h for x < 0, with h = Phi(-|x|) = erfc(z) / 2, z = |x| / sqrt 2:
// both sides free of cancellation.  erfc follows Abramowitz and Stegun,
// Handbook of Mathematical Functions, formula 7.1.26: erfc(z) ~ t (a1 + t
// (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) with t = 1 / (1 + p z), absolute
// error at most 1.5e-7 for z >= 0; here p z = (p / sqrt 2) |x|, the a_i are
// halved (exactly) to give h directly, and exp(-z^2) = 2^(-x^2 log2(e) / 2):
// one reciprocal, one exp2 and no branches, where the math library's erff
// is a long branchy sequence.  +inf gives +inf, -inf gives NaN (x * Phi(x)
// in IEEE arithmetic) and NaN stays NaN.
struct GeluErf {
    static constexpr float kP = 0.3275911f * 0.70710678118654752f;
    static constexpr float kE = -0.72134752044448170f;          // -log2(e) / 2
    static constexpr float kA1 = 0.5f * 0.254829592f, kA2 = 0.5f * -0.284496736f,
                           kA3 = 0.5f * 1.421413741f, kA4 = 0.5f * -1.453152027f,
                           kA5 = 0.5f * 1.061405429f;
};

// Keeps the compiler's scheduler from moving instructions across this
// point (no instruction is emitted).
__device__ __forceinline__ void sched_fence()
{
    __builtin_amdgcn_sched_barrier(0);
}

// N values at once, each step over all of them before the next, so that
// the reciprocal and exp2 latencies of one value overlap the others' work.
template <int N>
__device__ __forceinline__ void gelu_erf_n(float (&v)[N])
{
    float t[N], e[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        t[i] = __builtin_amdgcn_rcpf(fmaf(fabsf(v[i]), GeluErf::kP, 1.0f));
#pragma unroll
    for (int i = 0; i < N; ++i)
        e[i] = __builtin_amdgcn_exp2f(GeluErf::kE * v[i] * v[i]);
    if (N > 1)
        sched_fence();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float q = fmaf(t[i], GeluErf::kA5, GeluErf::kA4);
        q = fmaf(t[i], q, GeluErf::kA3);
        q = fmaf(t[i], q, GeluErf::kA2);
        q = fmaf(t[i], q, GeluErf::kA1);
        q *= t[i];
        const float h = q * e[i];                  // Phi(-|x|)
        const float g = fmaf(-q, e[i], 1.0f);      // 1 - h
        v[i] *= v[i] >= 0.0f ? g : h;
    }
}

__device__ __forceinline__ float gelu_erf(float x)
{
    float v[1] = {x};
    gelu_erf_n<1>(v);
    return v[0];
}

// GELU with the tanh approximation of the normal CDF:
// (1 + tanh(y)) / 2 with y = sqrt(2/pi) (x + 0.044715 x^3).  Uses the exact
// identity (1 + tanh(y)) / 2 = 1 / (1 + exp(-2y)), which has no
// cancellation; exp(-2y) = 2^(-2y log2(e)).
template <int N>
__device__ __forceinline__ void gelu_tanh_n(float (&v)[N])
{
    float e[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float y = 0.79788456080286536f * fmaf(0.044715f * v[i], v[i] * v[i], v[i]);
        e[i] = __builtin_amdgcn_exp2f(-2.8853900817779268f * y);
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = v[i] * __builtin_amdgcn_rcpf(1.0f + e[i]);
}

__device__ __forceinline__ float gelu_tanh(float x)
{
    float v[1] = {x};
    gelu_tanh_n<1>(v);
    return v[0];
}

// The activation on N values; ACT is a compile-time dg_act.
template <int32_t ACT, int N>
__device__ __forceinline__ void activate_n(float (&v)[N])
{
    if constexpr (ACT == ACT_GELU_ERF)
        gelu_erf_n<N>(v);
    else if constexpr (ACT == ACT_GELU_TANH)
        gelu_tanh_n<N>(v);
}

// The activation on N values, act a run-time (uniform) dg_act.
template <int N>
__device__ __forceinline__ void activate_n(float (&v)[N], int32_t act)
{
    if (act == ACT_GELU_ERF)
        gelu_erf_n<N>(v);
    else if (act == ACT_GELU_TANH)
        gelu_tanh_n<N>(v);
}

__device__ __forceinline__ float activate(float x, int32_t act)
{
    if (act == ACT_GELU_ERF)
        return gelu_erf(x);
    if (act == ACT_GELU_TANH)
        return gelu_tanh(x);
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
        v = fmaf(g.beta, load_as_f32(g.C, g.c_type, ci), v);
    }
    if (g.bias)
        v += load_as_f32(g.bias, g.bias_type, n);
    return activate(v, g.act);
}

__device__ __forceinline__ void store_c(const GemmArgs &g, int64_t b, int64_t m, int64_t n,
                                        float v)
{
    int64_t ci = b * g.sc + elem_offset(g.c_col, g.ldc, m, n);
    if (g.c_type == DT_BF16)
        ((uint16_t *)g.C)[ci] = f32_to_bf16(v);
    else if (g.c_type == DT_F16)
        ((uint16_t *)g.C)[ci] = f32_to_f16(v);
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
