/*
 * CPU oracle for the dense GEMM  C = act(alpha * A.B + beta * C_in + bias).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file.  It shares no source,
 * header, helper or table with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes, and where the pages define it:
 *   - the product C = alpha*A*B + beta*C ("La GEMM, de zero a cuBLAS",
 *     section 2.1, and the alpha*acc + beta*C store of its kernels in
 *     sections 2.2 and 2.4);
 *   - accumulation first, epilogue (alpha, beta*C, bias, activation) after
 *     the K loop, then the cast to the output dtype ("Skill: Write a Triton
 *     GEMM Kernel", Required reasoning process steps 4 and 6, Common failure
 *     modes on alpha/beta; "GEMM Kernel Optimization", Core Technique
 *     step 4);
 *   - batch strides per operand, stride 0 broadcasting an operand ("Skill:
 *     Write a Triton GEMM Kernel", Correctness requirements);
 *   - the reference is computed on the CPU in float64 ("Skill: Write a
 *     Triton GEMM Kernel", Required reasoning process step 8);
 *   - inputs in fp32, bf16 or fp16 ("Skill: Write a Triton GEMM Kernel",
 *     Inputs the agent should gather first: input dtype), decoded exactly;
 *     outputs rounded to nearest, ties to even, into fp32, bf16 or fp16.
 *
 * Readings where the pages are silent: the epilogue order is
 * act(alpha*acc + beta*c + bias); beta == 0 means C_in is not read;
 * alpha == 0 means A and B are not read; K == 0 gives acc = 0; GELU is the
 * exact erf form, with the tanh form as a second choice; rounding to the
 * output dtype is round-to-nearest-even.
 *
 * The sum over k is a plain ascending loop in double, compiled with
 * -ffp-contract=off so that every step is a separate multiply and add.
 * Each output element is computed by exactly one thread, so the result does
 * not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes used by this file's entry points */
#define OR_F32 0
#define OR_BF16 1
#define OR_F16 2
/* activation codes */
#define OR_ACT_NONE 0
#define OR_ACT_GELU_ERF 1
#define OR_ACT_GELU_TANH 2

typedef struct {
    int64_t M, N, K, batch;
    int32_t a_type, b_type, c_type, bias_type;
    int32_t a_col, b_col, c_col;       /* 1 = column-major */
    int64_t lda, ldb, ldc;
    int64_t stride_a, stride_b, stride_c;
    double alpha, beta;
    int32_t has_bias, act;
} oracle_problem;

/* ---- bf16 decode: the 16 stored bits are the top half of an fp32 ------- */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- fp16 decode: IEEE 754 binary16, 1 sign bit, 5 exponent bits (bias
 * 15), 10 fraction bits.  Exponent field 0 holds zero and the subnormals
 * fraction * 2^-24; field 31 holds infinities and NaNs; otherwise the value
 * is (1024 + fraction) * 2^(field - 25).  Every value is exact in double. */
static double f16_bits_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int field = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (field == 0)
        v = ldexp((double)frac, -24);
    else if (field == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), field - 25);
    return sign ? -v : v;
}

double oracle_f16_to_double(uint16_t h) { return f16_bits_to_double(h); }

static double load_value(const void *base, int32_t type, int64_t idx)
{
    if (type == OR_F32)
        return (double)((const float *)base)[idx];
    if (type == OR_F16)
        return f16_bits_to_double(((const uint16_t *)base)[idx]);
    return bf16_bits_to_double(((const uint16_t *)base)[idx]);
}

/* ---- bf16 encode: round a double to the nearest bf16, ties to even -----
 * bf16 has 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits.
 * Normal numbers in [2^e, 2^(e+1)) are spaced 2^(e-7) apart; below 2^-126
 * (subnormals) the spacing is 2^-133.  The two candidates are the
 * neighbours lo <= |x| < hi = lo + spacing; the nearer one wins and a tie
 * goes to the one with an even significand.  Anything at or above the
 * midpoint between the largest finite value and 2^128 becomes infinity.  */
uint16_t oracle_round_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double ax = fabs(x);
    /* largest finite bf16 = (2 - 2^-7) * 2^127; midpoint to 2^128 */
    double overflow_mid = ldexp(2.0, 127) - ldexp(1.0, 119);
    if (ax >= overflow_mid)
        return (uint16_t)(sign | 0x7F80u);
    if (ax == 0.0)
        return sign;
    int e;
    (void)frexp(ax, &e);            /* ax = f * 2^e, f in [0.5, 1) */
    int exp_unbiased = e - 1;       /* ax in [2^(e-1), 2^e) */
    if (exp_unbiased < -126)
        exp_unbiased = -126;        /* subnormal range shares the 2^-133 spacing */
    double spacing = ldexp(1.0, exp_unbiased - 7);
    double q = floor(ax / spacing); /* exact: division by a power of two */
    double lo = q * spacing;
    double hi = lo + spacing;
    double dlo = ax - lo, dhi = hi - ax;
    double pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (fmod(q, 2.0) == 0.0) ? lo : hi;
    /* pick is exactly representable in bf16, hence in fp32: take the top
     * 16 bits of its fp32 encoding. */
    float pf = (float)pick;
    uint32_t u;
    memcpy(&u, &pf, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* ---- fp16 encode: round a double to the nearest binary16, ties to even --
 * Normal numbers in [2^e, 2^(e+1)), e >= -14, are spaced 2^(e-10) apart;
 * below 2^-14 (subnormals) the spacing is 2^-24.  As for bf16, the nearer
 * of the two neighbours lo <= |x| < lo + spacing wins and a tie goes to the
 * even significand.  The largest finite value is (2 - 2^-10) * 2^15 =
 * 65504; at or above the midpoint 65520 between it and 2^16 the result is
 * infinity.  NaN becomes the quiet NaN 0x7E00 with its sign. */
uint16_t oracle_round_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00u);
    double ax = fabs(x);
    if (ax >= 65520.0)
        return (uint16_t)(sign | 0x7C00u);
    if (ax == 0.0)
        return sign;
    int e;
    (void)frexp(ax, &e);            /* ax in [2^(e-1), 2^e) */
    int exp_unbiased = e - 1;
    if (exp_unbiased < -14)
        exp_unbiased = -14;         /* subnormal range shares the 2^-24 spacing */
    double spacing = ldexp(1.0, exp_unbiased - 10);
    double q = floor(ax / spacing); /* exact: division by a power of two */
    double lo = q * spacing;
    double hi = lo + spacing;
    double dlo = ax - lo, dhi = hi - ax;
    double pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (fmod(q, 2.0) == 0.0) ? lo : hi;
    /* encode the (exactly representable) pick */
    if (pick < ldexp(1.0, -14))                       /* zero or subnormal */
        return (uint16_t)(sign | (uint16_t)(pick / ldexp(1.0, -24)));
    (void)frexp(pick, &e);
    int E = e - 1;                                    /* pick in [2^E, 2^(E+1)) */
    uint16_t frac = (uint16_t)((pick / ldexp(1.0, E) - 1.0) * 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | frac);
}

/* ---- activation --------------------------------------------------------
 * GELU(x) = x * Phi(x), Phi the standard normal CDF = (1 + erf(x/sqrt2))/2.
 * The tanh form replaces Phi by (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))/2. */
double oracle_act(double x, int32_t act)
{
    if (act == OR_ACT_GELU_ERF)
        return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    if (act == OR_ACT_GELU_TANH) {
        double inner = sqrt(2.0 / acos(-1.0)) * (x + 0.044715 * x * x * x);
        return 0.5 * x * (1.0 + tanh(inner));
    }
    return x;
}

static int64_t offset_of(int32_t col_major, int64_t ld, int64_t r, int64_t c)
{
    return col_major ? c * ld + r : r * ld + c;
}

/* One output element (b, i, j). */
static void one_element(const oracle_problem *p, const void *A, const void *B,
                        const void *Cin, const void *bias,
                        int64_t b, int64_t i, int64_t j,
                        double *ref, double *mag, void *out, int64_t out_idx)
{
    double acc = 0.0, amag = 0.0;
    if (p->alpha != 0.0) {
        int64_t abase = b * p->stride_a, bbase = b * p->stride_b;
        for (int64_t k = 0; k < p->K; ++k) {
            double a = load_value(A, p->a_type, abase + offset_of(p->a_col, p->lda, i, k));
            double w = load_value(B, p->b_type, bbase + offset_of(p->b_col, p->ldb, k, j));
            double prod = a * w;
            acc = acc + prod;
            amag = amag + fabs(a) * fabs(w);
        }
    }
    double c = 0.0;
    if (p->beta != 0.0)
        c = load_value(Cin, p->c_type, b * p->stride_c + offset_of(p->c_col, p->ldc, i, j));
    double bj = 0.0;
    if (p->has_bias)
        bj = load_value(bias, p->bias_type, j);
    double pre = p->alpha * acc + p->beta * c + bj;
    double v = oracle_act(pre, p->act);
    ref[out_idx] = v;
    mag[out_idx] = fabs(p->alpha) * amag + fabs(p->beta) * fabs(c) + fabs(bj);
    if (p->c_type == OR_F32)
        ((float *)out)[out_idx] = (float)v;
    else if (p->c_type == OR_F16)
        ((uint16_t *)out)[out_idx] = oracle_round_f16(v);
    else
        ((uint16_t *)out)[out_idx] = oracle_round_bf16(v);
}

static void set_threads(int32_t nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Whole problem.  ref, mag (double) and out (output dtype) are dense
 * [batch][M][N] arrays, independent of C's own layout. */
int oracle_gemm(const oracle_problem *p, const void *A, const void *B,
                const void *Cin, const void *bias,
                double *ref, double *mag, void *out, int32_t nthreads)
{
    if (!p || p->M < 0 || p->N < 0 || p->K < 0 || p->batch < 0)
        return 1;
    set_threads(nthreads);
    int64_t rows = p->batch * p->M;
    int64_t bi;
#pragma omp parallel for schedule(static)
    for (bi = 0; bi < rows; ++bi) {
        int64_t b = bi / p->M, i = bi % p->M;
        for (int64_t j = 0; j < p->N; ++j)
            one_element(p, A, B, Cin, bias, b, i, j, ref, mag, out, bi * p->N + j);
    }
    return 0;
}

/* Selected elements (pb[t], pi[t], pj[t]) for t < npts; ref/mag/out are
 * indexed by t.  Used for sampled checks of problems too large to
 * evaluate in full. */
int oracle_gemm_points(const oracle_problem *p, const void *A, const void *B,
                       const void *Cin, const void *bias,
                       const int64_t *pb, const int64_t *pi, const int64_t *pj,
                       int64_t npts, double *ref, double *mag, void *out,
                       int32_t nthreads)
{
    if (!p || npts < 0)
        return 1;
    set_threads(nthreads);
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < npts; ++t)
        one_element(p, A, B, Cin, bias, pb[t], pi[t], pj[t], ref, mag, out, t);
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
