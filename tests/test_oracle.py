"""Pins of the CPU oracle against values fixed by the mathematics.

None of these compares the oracle with itself: expected values come from
exact integer / rational arithmetic written independently here, closed forms
(identity, permutation, rank one, alpha = 0, beta = 0), an independent
library product (numpy float64 matmul), textbook standard-normal values and
hand-worked bf16 and fp16 rounding cases.  A dropped term, a wrong sign, a transposed
operand or a wrong layout index in the oracle fails at least one of them.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from conftest import read_golden

ORDERS = [W.ROW, W.COL]


def _log_f64(x, dtype):
    """Storage values -> float64 (bf16 / fp16 decoded exactly)."""
    if dtype == W.BF16:
        return oracle.bf16_bits_to_float(x)
    if dtype == W.F16:
        return oracle.f16_bits_to_float(x)
    return x.astype(np.float64)


def _run(p, x):
    return oracle.gemm(p, x.A, x.B, x.C, x.bias)


# ---------------------------------------------------------------------------
# P1: small-integer inputs, exact integer brute force
# ---------------------------------------------------------------------------
INT_CASES = []
for (ta, tc), (ao, bo, co) in itertools.product(
        [(W.F32, W.F32), (W.BF16, W.BF16), (W.BF16, W.F32), (W.F16, W.F16), (W.F16, W.F32)],
        itertools.product(ORDERS, ORDERS, ORDERS)):
    INT_CASES.append((ta, tc, ao, bo, co))


@pytest.mark.parametrize("ta,tc,ao,bo,co", INT_CASES)
def test_p1_small_integer_exact(ta, tc, ao, bo, co):
    # alpha = 1.5, beta = 0.5 are dyadic, so 2*out is an exact integer.
    for (M, N, K, batch, bias) in [(5, 7, 3, 1, False), (9, 4, 11, 3, True), (3, 6, 17, 2, True)]:
        p = W.Problem(name="int", M=M, N=N, K=K, batch=batch, a_type=ta, b_type=ta, c_type=tc,
                      a_order=ao, b_order=bo, c_order=co, alpha=1.5, beta=0.5,
                      has_bias=bias, bias_type=ta, seed=7)
        x = W.make_inputs(p, small_int=True)
        ref, mag, out = _run(p, x)
        A = _log_f64(x.A_log, ta).astype(np.int64)
        B = _log_f64(x.B_log, ta).astype(np.int64)
        C = _log_f64(x.C_log, tc).astype(np.int64)
        bias_v = _log_f64(x.bias, ta).astype(np.int64) if bias else np.zeros(N, np.int64)
        for b in range(batch):
            prod = np.zeros((M, N), np.int64)
            for i in range(M):          # plain triple loop over integers
                for j in range(N):
                    s = 0
                    for k in range(K):
                        s += int(A[b][i][k]) * int(B[b][k][j])
                    prod[i, j] = s
            twice = 3 * prod + C[b] + 2 * bias_v[None, :]
            assert np.array_equal(ref[b] * 2, twice.astype(np.float64))
            if tc == W.F32:
                assert np.array_equal(out[b].astype(np.float64) * 2, twice.astype(np.float64))
            else:
                # |2 out| <= 3*4*17 + 2 + 4 < 256: every half-integer result
                # has at most 8 significant bits, so bf16 (and fp16) holds it exactly.
                assert np.array_equal(_log_f64(out[b], tc) * 2, twice.astype(np.float64))


def test_p1_integer_larger_k_f32():
    # |acc| <= 4K = 8192 < 2^24: every intermediate is exact in any precision.
    p = W.Problem(name="int", M=33, N=17, K=2048, alpha=1.5, beta=0.5, seed=3)
    x = W.make_inputs(p, small_int=True)
    ref, mag, out = _run(p, x)
    A = x.A_log[0].astype(np.int64)
    B = x.B_log[0].astype(np.int64)
    C = x.C_log[0].astype(np.int64)
    twice = 3 * (A @ B) + C
    assert np.array_equal(ref[0] * 2, twice.astype(np.float64))
    assert np.array_equal(out[0].astype(np.float64) * 2, twice.astype(np.float64))


# ---------------------------------------------------------------------------
# P2: tiny random problems, exact rationals, every layout and broadcast
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ao,bo,co", list(itertools.product(ORDERS, ORDERS, ORDERS)))
@pytest.mark.parametrize("bcast", ["none", "a", "b"])
def test_p2_exact_rational(ao, bo, co, bcast):
    rng = np.random.default_rng(11)
    for trial in range(4):
        M, N, K = (int(v) for v in rng.integers(1, 5, size=3))
        batch = int(rng.integers(1, 4))
        pad = int(rng.integers(0, 3))
        kw = {}
        if bcast == "a":
            kw["stride_a"] = 0
        if bcast == "b":
            kw["stride_b"] = 0
        lda = (K if ao == W.ROW else M) + pad
        ldb = (N if bo == W.ROW else K) + pad
        ldc = (N if co == W.ROW else M) + pad
        p = W.Problem(name="frac", M=M, N=N, K=K, batch=batch, a_order=ao, b_order=bo,
                      c_order=co, lda=lda, ldb=ldb, ldc=ldc, alpha=-0.75, beta=1.25,
                      has_bias=True, bias_type=W.F32, seed=100 + trial, **kw)
        x = W.make_inputs(p, fill=float("nan"))
        ref, mag, out = _run(p, x)
        for b in range(batch):
            Ab = x.A_log[0 if bcast == "a" else b]
            Bb = x.B_log[0 if bcast == "b" else b]
            for i in range(M):
                for j in range(N):
                    s = Fraction(0)
                    for k in range(K):
                        s += Fraction(float(Ab[i][k])) * Fraction(float(Bb[k][j]))
                    exact = (Fraction(-3, 4) * s + Fraction(5, 4) * Fraction(float(x.C_log[b][i][j]))
                             + Fraction(float(x.bias[j])))
                    err = abs(Fraction(ref[b, i, j]) - exact)
                    assert err <= Fraction(8, 2 ** 53) * Fraction(mag[b, i, j]), (b, i, j)
                    assert out[b, i, j] == np.float32(float(exact)) or \
                        abs(float(out[b, i, j]) - float(exact)) <= 2 ** -23 * abs(float(exact))


# ---------------------------------------------------------------------------
# P3 identity, P4 permutation, P6 rank one
# ---------------------------------------------------------------------------
def _dyadic(rng, shape):
    """Values k / 2^12 with |k| <= 2^12: sums of a few products stay exact."""
    return (rng.integers(-4096, 4097, size=shape) / 4096.0).astype(np.float32)


def _custom_inputs(p, A_log, B_log, C_log, bias=None):
    A = W.lay_out(A_log, p.a_order, p.lda_, p.stride_a_, p.buffer_elems("a"), p.a_type)
    B = W.lay_out(B_log, p.b_order, p.ldb_, p.stride_b_, p.buffer_elems("b"), p.b_type)
    C = W.lay_out(C_log, p.c_order, p.ldc_, p.stride_c_, p.buffer_elems("c"), p.c_type)
    return A, B, C, bias


@pytest.mark.parametrize("ao,bo,co", list(itertools.product(ORDERS, ORDERS, ORDERS)))
def test_p3_identity(ao, bo, co):
    rng = np.random.default_rng(5)
    M, N = 13, 9
    p = W.Problem(name="id", M=M, N=N, K=M, a_order=ao, b_order=bo, c_order=co,
                  alpha=1.5, beta=0.5)
    B_log = _dyadic(rng, (1, M, N))
    C_log = _dyadic(rng, (1, M, N))
    A_log = np.eye(M, dtype=np.float32)[None]
    A, B, C, _ = _custom_inputs(p, A_log, B_log, C_log)
    ref, mag, out = oracle.gemm(p, A, B, C)
    expect = 1.5 * B_log[0].astype(np.float64) + 0.5 * C_log[0].astype(np.float64)
    assert np.array_equal(ref[0], expect)


@pytest.mark.parametrize("ao,bo", list(itertools.product(ORDERS, ORDERS)))
def test_p4_permutation(ao, bo):
    rng = np.random.default_rng(6)
    M, N = 11, 7
    sigma = rng.permutation(M)
    A_log = np.zeros((1, M, M), np.float32)
    A_log[0, np.arange(M), sigma] = 1.0      # row i of A picks row sigma[i] of B
    B_log = _dyadic(rng, (1, M, N))
    C_log = np.zeros((1, M, N), np.float32)
    p = W.Problem(name="perm", M=M, N=N, K=M, a_order=ao, b_order=bo, alpha=2.0, beta=0.0)
    A, B, C, _ = _custom_inputs(p, A_log, B_log, C_log)
    ref, mag, out = oracle.gemm(p, A, B, C)
    assert np.array_equal(ref[0], 2.0 * B_log[0][sigma].astype(np.float64))
    # the magnitude scale is exactly |alpha| |B[sigma]| here
    assert np.array_equal(mag[0], 2.0 * np.abs(B_log[0][sigma]).astype(np.float64))


def test_p6_rank_one_k1_and_outer_products():
    rng = np.random.default_rng(8)
    # K = 1: one product per element
    M, N = 6, 5
    p = W.Problem(name="k1", M=M, N=N, K=1, alpha=0.25, beta=-2.0)
    u = _dyadic(rng, (1, M, 1))
    v = _dyadic(rng, (1, 1, N))
    C_log = _dyadic(rng, (1, M, N))
    A, B, C, _ = _custom_inputs(p, u, v, C_log)
    ref, _, _ = oracle.gemm(p, A, B, C)
    exp = 0.25 * (u[0].astype(np.float64) @ v[0].astype(np.float64)) - 2.0 * C_log[0]
    assert np.array_equal(ref[0], exp)
    # A = u x^T, B = y v^T  =>  A B = (x . y) u v^T
    K = 5
    ui = rng.integers(-3, 4, size=M).astype(np.float64)
    xi = rng.integers(-3, 4, size=K).astype(np.float64)
    yi = rng.integers(-3, 4, size=K).astype(np.float64)
    vi = rng.integers(-3, 4, size=N).astype(np.float64)
    p = W.Problem(name="r1", M=M, N=N, K=K, a_order=W.COL, b_order=W.ROW, alpha=1.0, beta=0.0)
    A_log = np.outer(ui, xi).astype(np.float32)[None]
    B_log = np.outer(yi, vi).astype(np.float32)[None]
    A, B, C, _ = _custom_inputs(p, A_log, B_log, np.zeros((1, M, N), np.float32))
    ref, _, _ = oracle.gemm(p, A, B, C)
    assert np.array_equal(ref[0], float(xi @ yi) * np.outer(ui, vi))


# ---------------------------------------------------------------------------
# P5: alpha = 0 reads neither A nor B; beta = 0 does not read C
# ---------------------------------------------------------------------------
def test_p5_alpha_zero_and_beta_zero():
    rng = np.random.default_rng(9)
    M, N, K = 7, 6, 5
    p = W.Problem(name="a0", M=M, N=N, K=K, alpha=0.0, beta=0.5, has_bias=True)
    A_log = np.full((1, M, K), np.nan, np.float32)
    B_log = np.full((1, K, N), np.nan, np.float32)
    C_log = _dyadic(rng, (1, M, N))
    bias = _dyadic(rng, (N,))
    A, B, C, _ = _custom_inputs(p, A_log, B_log, C_log)
    ref, mag, _ = oracle.gemm(p, A, B, C, bias)
    assert np.array_equal(ref[0], 0.5 * C_log[0].astype(np.float64) + bias[None, :])
    # A and B may even be absent
    ref2, _, _ = oracle.gemm(p, None, None, C, bias)
    assert np.array_equal(ref2, ref)
    # beta = 0: NaN in C must not reach the result
    p = W.Problem(name="b0", M=M, N=N, K=K, alpha=1.0, beta=0.0)
    A_log = _dyadic(rng, (1, M, K))
    B_log = _dyadic(rng, (1, K, N))
    C_log = np.full((1, M, N), np.nan, np.float32)
    A, B, C, _ = _custom_inputs(p, A_log, B_log, C_log)
    ref, _, _ = oracle.gemm(p, A, B, C)
    assert not np.isnan(ref).any()
    assert np.array_equal(ref[0], A_log[0].astype(np.float64) @ B_log[0].astype(np.float64))


def test_k_zero_and_empty():
    p = W.Problem(name="k0", M=3, N=4, K=0, alpha=1.0, beta=2.0, has_bias=True, lda=1, ldb=4)
    C_log = np.arange(12, dtype=np.float32).reshape(1, 3, 4)
    bias = np.array([1, 2, 3, 4], np.float32)
    C = W.lay_out(C_log, p.c_order, p.ldc_, p.stride_c_, p.buffer_elems("c"), p.c_type)
    ref, mag, out = oracle.gemm(p, np.zeros(1, np.float32), np.zeros(1, np.float32), C, bias)
    assert np.array_equal(ref[0], 2.0 * C_log[0] + bias[None, :])
    p = W.Problem(name="m0", M=0, N=4, K=3)
    ref, mag, out = oracle.gemm(p, np.zeros(1, np.float32), np.zeros(12, np.float32),
                                np.zeros(1, np.float32))
    assert ref.shape == (1, 0, 4)


# ---------------------------------------------------------------------------
# P7: independent float64 library product at a ragged size
# ---------------------------------------------------------------------------
def test_p7_numpy_float64_cross_check():
    p = W.Problem(name="np", M=257, N=259, K=263, a_order=W.COL, b_order=W.ROW,
                  c_order=W.COL, alpha=0.7, beta=-1.3, seed=21)
    x = W.make_inputs(p)
    ref, mag, out = _run(p, x)
    A = x.A_log[0].astype(np.float64)
    B = x.B_log[0].astype(np.float64)
    C = x.C_log[0].astype(np.float64)
    exp = 0.7 * (A @ B) + (-1.3) * C
    assert np.all(np.abs(ref[0] - exp) <= 1e-12 * mag[0])
    assert np.allclose(mag[0], 0.7 * (np.abs(A) @ np.abs(B)) + 1.3 * np.abs(C), rtol=1e-12)


def test_bf16_inputs_decoded_exactly():
    p = W.Problem(name="bf", M=31, N=29, K=37, a_type=W.BF16, b_type=W.BF16, c_type=W.F32,
                  a_order=W.ROW, b_order=W.COL, dist_a=("normal", 1.0), dist_b=("normal", 1.0),
                  alpha=1.0, beta=0.0, seed=22)
    x = W.make_inputs(p)
    ref, mag, out = _run(p, x)
    # decode by an independent route: place the 16 bits on top of a float32
    A = np.frombuffer((x.A_log.astype(np.uint32) << 16).tobytes(), np.float32)
    B = np.frombuffer((x.B_log.astype(np.uint32) << 16).tobytes(), np.float32)
    A = A.reshape(p.M, p.K).astype(np.float64)
    B = B.reshape(p.K, p.N).astype(np.float64)
    assert np.all(np.abs(ref[0] - A @ B) <= 1e-13 * mag[0])


def test_points_match_full_evaluation():
    p = W.WORKLOADS["c1"]
    x = W.make_inputs(p)
    ref, mag, out = _run(p, x)
    pb, pi, pj = W.sample_points(p, 200)
    r2, m2, o2 = oracle.gemm_points(p, x.A, x.B, x.C, x.bias, pb, pi, pj)
    assert np.array_equal(r2, ref[pb, pi, pj])
    assert np.array_equal(m2, mag[pb, pi, pj])
    assert np.array_equal(o2, out[pb, pi, pj])


def test_thread_count_does_not_change_result():
    p = W.Problem(name="thr", M=67, N=45, K=301, seed=4)
    x = W.make_inputs(p)
    r1 = oracle.gemm(p, x.A, x.B, x.C, nthreads=1)
    r4 = oracle.gemm(p, x.A, x.B, x.C, nthreads=4)
    for a, b in zip(r1, r4):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# P8: GELU
# ---------------------------------------------------------------------------
def test_p8_gelu_erf_normal_table():
    for xs, phis in read_golden("normal_cdf.txt"):
        x, phi = float(xs), float(phis)
        assert abs(oracle.act(x, "gelu_erf") - x * phi) <= 1e-11 * max(1.0, x)
        assert abs(oracle.act(-x, "gelu_erf") - (-x * (1.0 - phi))) <= 1e-11 * max(1.0, x)


@pytest.mark.parametrize("kind", ["gelu_erf", "gelu_tanh"])
def test_p8_gelu_invariants(kind):
    assert oracle.act(0.0, kind) == 0.0
    for x in np.linspace(-6, 6, 241):
        g = oracle.act(x, kind)
        # x Phi(x) - (-x)(Phi(-x)) = x (Phi(x) + 1 - Phi(x)) = x
        assert abs((g - oracle.act(-x, kind)) - x) <= 1e-14 * max(1.0, abs(x))
        assert (g >= 0) == (x >= 0) or abs(g) < 1e-300 or x < 0 and g <= 0
    assert abs(oracle.act(30.0, kind) - 30.0) < 1e-12
    assert abs(oracle.act(-30.0, kind)) < 1e-12
    assert oracle.act(3.0, "none") == 3.0


def test_p8_gelu_tanh_close_to_erf_form():
    # The tanh form approximates x Phi(x) to within a few 1e-4 everywhere;
    # a wrong constant or a dropped cubic term moves it far outside this.
    xs = np.linspace(-8, 8, 1601)
    d = max(abs(oracle.act(x, "gelu_tanh") - oracle.act(x, "gelu_erf")) for x in xs)
    assert d < 1e-3
    assert d > 1e-6     # and it is a different function


# The tanh form is x (1 + tanh y) / 2 with y = sqrt(2/pi) (x + 0.044715 x^3).
# Where tanh y takes a chosen value tau, it equals x (1 + tau) / 2 exactly;
# y = atanh(tau) = ln((1 + tau) / (1 - tau)) / 2 and the x with that y is the
# root of an increasing cubic, found here by bisection in 50-digit decimals.
# A slip in either constant moves tanh y off tau by about 1e-6 (0.0447 for
# 0.044715) or 1e-3 (0.8 for sqrt(2/pi)) and fails the 1e-13 check.
def _x_where_tanh_is(tau):
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    y = ((1 + Decimal(tau)) / (1 - Decimal(tau))).ln() / 2
    # sqrt(2/pi) to 40 digits from pi = 3.14159265358979323846264338327950288419
    pi = Decimal("3.14159265358979323846264338327950288419")
    s = (Decimal(2) / pi).sqrt()
    c = Decimal("0.044715")
    lo, hi = Decimal(-10), Decimal(10)
    for _ in range(200):
        mid = (lo + hi) / 2
        if s * (mid + c * mid ** 3) < y:
            lo = mid
        else:
            hi = mid
    return float((lo + hi) / 2)


@pytest.mark.parametrize("tau", [0.5, -0.5, 0.8, -0.8, 0.25, 0.95])
def test_p8_gelu_tanh_where_tanh_is_known(tau):
    x = _x_where_tanh_is(tau)
    want = x * (1.0 + tau) / 2.0          # 0.75 x at tau = 1/2
    got = oracle.act(x, "gelu_tanh")
    assert abs(got - want) <= 1e-13 * max(1.0, abs(x)), (tau, x, got, want)


def test_p8_gelu_tanh_high_precision_points():
    """Four points evaluated from the definition in 50-digit decimal
    arithmetic, tanh through exp (tanh y = (e^2y - 1) / (e^2y + 1)), held to
    the oracle within 1e-14 relative."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    pi = Decimal("3.14159265358979323846264338327950288419")
    s = (Decimal(2) / pi).sqrt()
    c = Decimal("0.044715")
    for xs in ("-2.75", "-0.3", "0.7", "1.9"):
        x = Decimal(xs)
        y = s * (x + c * x ** 3)
        e = (2 * y).exp()
        want = x * (1 + (e - 1) / (e + 1)) / 2
        got = oracle.act(float(x), "gelu_tanh")
        assert abs(Decimal(got) - want) <= Decimal("1e-14") * abs(want), (xs, got, want)


# ---------------------------------------------------------------------------
# P9: bf16 round to nearest even
# ---------------------------------------------------------------------------
def _parse_float(s):
    if s == "-0":
        return -0.0
    if s in ("inf", "-inf", "nan"):
        return float(s)
    return float.fromhex(s)


def test_p9_bf16_rne_table():
    rows = read_golden("bf16_rne.txt")
    assert len(rows) >= 20
    for row in rows:
        x, expect = _parse_float(row[0]), int(row[1], 16)
        assert oracle.round_bf16(x) == expect, (row[0], hex(oracle.round_bf16(x)), row[1])


def test_p9_bf16_output_rounding_in_gemm():
    # 1 * 1 + (2^-8) * 1 = 1 + 2^-8: the tie case, must round to even (1.0)
    p = W.Problem(name="tie", M=1, N=1, K=2, a_type=W.BF16, b_type=W.BF16, c_type=W.BF16)
    A = np.array([0x3F80, 0x3B80], np.uint16)     # 1.0, 2^-8
    B = np.array([0x3F80, 0x3F80], np.uint16)     # 1.0, 1.0
    C = np.zeros(1, np.uint16)
    ref, mag, out = oracle.gemm(p, A, B, C)
    assert ref[0, 0, 0] == 1.0 + 2 ** -8
    assert out[0, 0, 0] == 0x3F80


# ---------------------------------------------------------------------------
# P10: fp16 inputs and output ("Skill: Write a Triton GEMM Kernel", Inputs the
# agent should gather first: input dtype; fp16 is the dtype of the pages'
# allclose check)
# ---------------------------------------------------------------------------
def test_p10_f16_rne_table():
    rows = read_golden("f16_rne.txt")
    assert len(rows) >= 25
    for row in rows:
        x, expect = _parse_float(row[0]), int(row[1], 16)
        assert oracle.round_f16(x) == expect, (row[0], hex(oracle.round_f16(x)), row[1])


def test_p10_f16_rne_matches_numpy_on_random_doubles():
    # numpy's float64 -> float16 conversion rounds to nearest even straight
    # from double (one rounding): an independent implementation of the format
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        rng.uniform(-70000, 70000, 500),
        # every midpoint between adjacent fp16 values of one binade, and next to it
        (np.arange(1024, 2048) + 0.5) * 2.0 ** -10,
        np.nextafter((np.arange(1024, 2048) + 0.5) * 2.0 ** -10, 0),
        (np.arange(0, 1024) + 0.5) * 2.0 ** -24,
    ])
    with np.errstate(over="ignore"):          # values past 65520 round to infinity on purpose
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.round_f16(x) for x in xs], np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float.hex(float(xs[i])), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_p10_f16_decode_every_pattern():
    # every finite bit pattern, decoded through numpy's float16 as the
    # independent route; NaN patterns decode to NaN, infinities keep their sign
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_float(b) for b in bits[::7]])
    w = want[::7]
    same = (got == w) | (np.isnan(got) & np.isnan(w))
    assert same.all()
    assert oracle.f16_to_float(0x0001) == 2.0 ** -24
    assert oracle.f16_to_float(0x7BFF) == 65504.0
    assert oracle.f16_to_float(0xFC00) == -math.inf


def test_p10_f16_inputs_decoded_exactly():
    p = W.Problem(name="h", M=31, N=29, K=37, a_type=W.F16, b_type=W.F16, c_type=W.F32,
                  a_order=W.ROW, b_order=W.COL, dist_a=("normal", 1.0), dist_b=("normal", 1.0),
                  alpha=1.0, beta=0.0, seed=23)
    x = W.make_inputs(p)
    ref, mag, out = _run(p, x)
    # decode by an independent route: expand each half to float32 by
    # rebuilding sign, exponent and fraction with integer arithmetic
    def expand(h):
        h = h.astype(np.int64)
        sign = np.where(h >> 15, -1.0, 1.0)
        e = (h >> 10) & 31
        f = h & 1023
        return sign * np.where(e == 0, f * 2.0 ** -24, (1024 + f) * 2.0 ** (e - 25))
    A = expand(x.A_log.reshape(p.M, p.K))
    B = expand(x.B_log.reshape(p.K, p.N))
    assert np.all(np.abs(ref[0] - A @ B) <= 1e-13 * mag[0])


def test_p10_f16_output_rounding_in_gemm():
    # 1 * 1 + 2^-11 * 1 is the tie between 1 and 1 + 2^-10: even (1.0) wins;
    # 1 + 2^-10 + 2^-11 ties between odd 1 + 2^-10 and even 1 + 2^-9
    p = W.Problem(name="tie", M=1, N=2, K=3, a_type=W.F16, b_type=W.F16, c_type=W.F16,
                  b_order=W.COL)
    A = np.array([0x3C00, 0x1000, 0x1400], np.uint16)     # 1, 2^-11, 2^-10
    B = np.array([0x3C00, 0x3C00, 0x0000,                  # column 0: 1, 1, 0
                  0x3C00, 0x3C00, 0x3C00], np.uint16)      # column 1: 1, 1, 1
    C = np.zeros(2, np.uint16)
    ref, mag, out = oracle.gemm(p, A, B, C)
    assert ref[0, 0, 0] == 1.0 + 2 ** -11 and out[0, 0, 0] == 0x3C00
    assert ref[0, 0, 1] == 1.0 + 2 ** -10 + 2 ** -11 and out[0, 0, 1] == 0x3C02


def test_p10_f16_overflow_to_infinity_in_gemm():
    # 255 * 255 + 255 * 2 = 65535 is above the 65520 midpoint: +inf; with
    # alpha = -1 the sign follows
    p = W.Problem(name="ovf", M=1, N=1, K=2, a_type=W.F16, b_type=W.F16, c_type=W.F16)
    A = np.array([0x5BF8, 0x5BF8], np.uint16)   # 255, 255
    B = np.array([0x5BF8, 0x4000], np.uint16)   # 255, 2
    ref, mag, out = oracle.gemm(p, A, B, np.zeros(1, np.uint16))
    assert ref[0, 0, 0] == 65535.0 and out[0, 0, 0] == 0x7C00
    ref, mag, out = oracle.gemm(p.replace(alpha=-1.0), A, B, np.zeros(1, np.uint16))
    assert out[0, 0, 0] == 0xFC00
