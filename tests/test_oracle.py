"""Pins of the CPU oracle to facts outside itself (runs without a GPU).

The oracle computes C[m][n] = sum_k A[m][k] * B[n][k] in fp64 (CuTe DSL Ampere
SGEMM example: module docstring, reference check in run(); CK Tile practice
GEMM README: "Host Matrix Creation", "Result Verification").  Each test below
checks it against something it does not share code with: a hand-worked
fixture, exact integer arithmetic in Python, closed forms, invariants of the
definition, exact rational arithmetic, numpy's BLAS, and numpy's IEEE
conversions.  The last test plants plausible mistakes and shows the pins
catch them.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from oracle import compare

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [(a, b) for a in "km" for b in "kn"]


def _oracle_logical(a_log, b_log, a_major="k", b_major="k", in_type="f32", threads=1, rows=None,
                    ld_extra=0):
    """Run the oracle on logical fp32 matrices laid out in the given majors."""
    M, K = a_log.shape
    N = b_log.shape[0]
    at, bt = gi.cast(a_log, in_type), gi.cast(b_log, in_type)
    eb = gi.ELEM_BYTES[in_type]
    lda = gi.min_ld(M if a_major == "m" else K, eb) + ld_extra
    ldb = gi.min_ld(N if b_major == "n" else K, eb) + ld_extra
    A = gi.store(at, a_major == "m", lda)
    B = gi.store(bt, b_major == "n", ldb)
    return oracle.gemm_ref(M, N, K, a_major, b_major, in_type, A, lda, B, ldb, rows=rows,
                           threads=threads)


def _python_exact(a_log, b_log):
    """Exact sum with Python integers / Fractions, no floating point."""
    M, K = a_log.shape
    N = b_log.shape[0]
    out = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(a_log[m, k])) * Fraction(float(b_log[n, k]))
            out[m][n] = s
    return out


# ---------------------------------------------------------------- fixtures

def test_hand_worked_fixture_all_layouts():
    with open(os.path.join(GOLDEN, "hand_worked_2x2.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        a = np.array(case["A"], dtype=np.float32)
        b = np.array(case["B"], dtype=np.float32)
        want = np.array(case["C"], dtype=np.float64)
        for am, bm in LAYOUTS:
            for ld_extra in (0, 4):
                got = _oracle_logical(a, b, am, bm, ld_extra=ld_extra)
                assert np.array_equal(got, want), (am, bm, got, want)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("in_type", ["f32", "f16", "bf16"])
def test_bruteforce_tiny_all_layouts(in_type):
    """Every M, N, K in {0,1,2,3,5} and every layout, integer inputs, against
    exact Python integer arithmetic."""
    rng = np.random.Generator(np.random.PCG64(7))
    sizes = [0, 1, 2, 3, 5]
    for M, N, K in itertools.product(sizes, sizes, sizes):
        a = rng.integers(-5, 6, size=(M, K)).astype(np.float32)
        b = rng.integers(-5, 6, size=(N, K)).astype(np.float32)
        exact = [[sum(int(a[m, k]) * int(b[n, k]) for k in range(K)) for n in range(N)]
                 for m in range(M)]
        want = np.array(exact, dtype=np.float64).reshape(M, N)
        for am, bm in LAYOUTS:
            got = _oracle_logical(a, b, am, bm, in_type=in_type)
            assert got.shape == (M, N)
            assert np.array_equal(got, want), (M, N, K, am, bm)


def test_exact_within_rounding_bound_noninteger():
    """On random fp32 data the fp64 result is within K * 2^-53 * sum|a||b| of
    the exact rational sum (the only rounding is in the additions)."""
    rng = np.random.Generator(np.random.PCG64(11))
    for M, N, K in [(3, 4, 37), (2, 2, 200), (5, 1, 64)]:
        a = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
        b = rng.uniform(-1, 1, size=(N, K)).astype(np.float32)
        exact = _python_exact(a, b)
        got = _oracle_logical(a, b, "m", "n")
        for m in range(M):
            for n in range(N):
                bound = K * 2.0 ** -53 * float(np.sum(np.abs(a[m].astype(np.float64) *
                                                             b[n].astype(np.float64))))
                assert abs(Fraction(float(got[m, n])) - exact[m][n]) <= Fraction(bound)


def test_sequential_fp64_sum_bitwise():
    """Every element is one fp64 sum over k ascending, multiply and add as
    separate IEEE operations: a Python loop over floats (IEEE doubles, one
    rounding per operation) gives the same bits.  N = 11 and 6 leave column
    remainders after the oracle's groups of four."""
    rng = np.random.Generator(np.random.PCG64(13))
    for M, N, K, kind in [(5, 11, 67, "u11"), (3, 6, 130, "n01"), (2, 9, 1, "u11")]:
        a = gi.draw(rng, M, K, kind)
        b = gi.draw(rng, N, K, kind)
        got = _oracle_logical(a, b, "k", "n", threads=2)
        for m in range(M):
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s = s + float(a[m, k]) * float(b[n, k])
                assert got[m, n] == s, (M, N, K, m, n)
    # k ascending: 1 + 2^-61 rounds to 1, then -1 cancels it (a sum that adds
    # the first and last terms first keeps the 2^-61).
    a = np.array([[1.0, 2.0 ** -30, -1.0]], dtype=np.float32)
    b = np.array([[1.0, 2.0 ** -31, 1.0]] * 5, dtype=np.float32)
    assert np.all(_oracle_logical(a, b) == 0.0)


# ---------------------------------------------------------------- closed forms

def test_closed_forms():
    M, N, K = 7, 5, 13
    # all ones: C = K
    c = _oracle_logical(np.ones((M, K), np.float32), np.ones((N, K), np.float32), "m", "k")
    assert np.all(c == K)
    # rank one: A[m,k] = u_m, B[n,k] = v_n  ->  C = K u_m v_n
    u = np.arange(1, M + 1, dtype=np.float32) - 3
    v = np.arange(1, N + 1, dtype=np.float32) * 2 - 5
    c = _oracle_logical(np.repeat(u[:, None], K, 1), np.repeat(v[:, None], K, 1), "k", "n")
    assert np.array_equal(c, K * np.outer(u, v).astype(np.float64))
    # A[m,k] = m, B = 1  ->  C[m,n] = m K
    c = _oracle_logical(np.repeat(np.arange(M, dtype=np.float32)[:, None], K, 1),
                        np.ones((N, K), np.float32), "m", "n")
    assert np.array_equal(c, np.repeat(np.arange(M)[:, None] * K, N, 1).astype(np.float64))


def test_identity_and_permutation():
    rng = np.random.Generator(np.random.PCG64(3))
    K = N = 9
    b = rng.uniform(-1, 1, size=(N, K)).astype(np.float32)
    eye = np.eye(K, dtype=np.float32)
    for am, bm in LAYOUTS:
        # A = I  ->  C[m,n] = B[n,m]
        c = _oracle_logical(eye, b, am, bm)
        assert np.array_equal(c, b.T.astype(np.float64))
        # A = P (a permutation matrix, A[m, p[m]] = 1)  ->  C[m,n] = B[n, p[m]]
        p = rng.permutation(K)
        P = np.zeros((K, K), np.float32)
        P[np.arange(K), p] = 1
        c = _oracle_logical(P, b, am, bm)
        assert np.array_equal(c, b[:, p].T.astype(np.float64))


# ---------------------------------------------------------------- invariants

def test_transpose_invariance_bitwise():
    """C^T = B A^T: swapping the operands transposes C exactly, since each
    element sees the same products in the same k order."""
    rng = np.random.Generator(np.random.PCG64(5))
    a = rng.uniform(-1, 1, size=(19, 33)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(23, 33)).astype(np.float32)
    for am, bm in LAYOUTS:
        c = _oracle_logical(a, b, am, bm)
        ct = _oracle_logical(b, a, "k" if bm == "k" else "m", "k" if am == "k" else "n")
        assert np.array_equal(c, ct.T)


def test_layout_invariance_bitwise():
    rng = np.random.Generator(np.random.PCG64(9))
    for in_type in ("f32", "f16", "bf16"):
        a = rng.standard_normal(size=(21, 40)).astype(np.float32)
        b = rng.standard_normal(size=(17, 40)).astype(np.float32)
        ref = _oracle_logical(a, b, "k", "k", in_type=in_type)
        for am, bm in LAYOUTS:
            for ld_extra in (0, 8):
                assert np.array_equal(_oracle_logical(a, b, am, bm, in_type=in_type,
                                                      ld_extra=ld_extra), ref)


def test_threads_and_row_subsets_bitwise():
    rng = np.random.Generator(np.random.PCG64(13))
    a = rng.uniform(-1, 1, size=(37, 50)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(29, 50)).astype(np.float32)
    one = _oracle_logical(a, b, "m", "k", threads=1)
    for t in (2, 3, 8, 64):
        assert np.array_equal(_oracle_logical(a, b, "m", "k", threads=t), one)
    for r0, r1 in [(0, 1), (5, 17), (36, 37), (10, 10)]:
        sub = _oracle_logical(a, b, "m", "k", threads=4, rows=(r0, r1))
        assert np.array_equal(sub, one[r0:r1])


# ---------------------------------------------------------------- library routine

def test_agrees_with_numpy_blas_fp64():
    rng = np.random.Generator(np.random.PCG64(17))
    a = rng.uniform(-1, 1, size=(130, 300)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(70, 300)).astype(np.float32)
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    got = _oracle_logical(a, b, "k", "n", threads=4)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= 1e-14


# ---------------------------------------------------------------- element formats

def test_decode_f16_all_patterns_vs_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode(bits, "f16")
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isnan(got[~fin]))
    assert oracle.decode(np.array([0x3C00, 0x0001, 0x8400, 0x7BFF], np.uint16), "f16").tolist() == \
        [1.0, 2.0 ** -24, -(2.0 ** -14), 65504.0]


def test_decode_bf16_all_patterns_vs_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.decode(bits, "bf16")
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert oracle.decode(np.array([0x3F80, 0xC000, 0x0001], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, 2.0 ** -133]


def _interesting_doubles(rng, n):
    x = rng.standard_normal(n) * np.exp2(rng.integers(-140, 20, n).astype(np.float64))
    return np.concatenate([x, [0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 1e30, -1e-45]])


def test_round_f32_and_f16_vs_numpy():
    rng = np.random.Generator(np.random.PCG64(21))
    x = _interesting_doubles(rng, 200000)
    assert np.array_equal(oracle.round_to(x, "f32").view(np.uint32),
                          x.astype(np.float32).view(np.uint32))
    # ties: a half-way double between two fp16 values rounds to the even one
    f16 = np.arange(0x0001, 0x7BFF, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = (np.arange(0x0001, 0x7BFF, 37, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    ties = (f16 + nxt) / 2
    x = np.concatenate([x[np.abs(x) < 1e6], ties, -ties])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.round_to(x, "f16"), want)


def _bf16_nearest_bruteforce(x):
    """Nearest bf16 by searching the neighbours of the truncated pattern with
    exact rational distances; ties go to the even pattern."""
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    f32 = np.float32(x)
    base = int(np.array([f32], np.float32).view(np.uint32)[0] >> 16)
    best = None
    for cand in range(max(base - 2, 0), base + 3):
        if (cand & 0x7F80) == 0x7F80:     # inf / nan patterns
            continue
        v = float(np.array([cand << 16], np.uint32).view(np.float32)[0])
        if (v < 0) != (x < 0) and v != 0:
            continue
        d = abs(Fraction(v) - Fraction(float(x)))
        key = (d, cand & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_round_bf16_vs_bruteforce():
    rng = np.random.Generator(np.random.PCG64(23))
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-130, 100, 3000).astype(np.float64))
    # exact ties between consecutive bf16 values, both parities
    k = rng.integers(0x0080, 0x7F00, 500).astype(np.uint32)
    lo = (k << 16).view(np.float32).astype(np.float64)
    hi = ((k + 1) << 16).view(np.float32).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, [1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]])
    got = oracle.round_to(x, "bf16")
    for xi, gi_ in zip(x, got):
        assert int(gi_) == _bf16_nearest_bruteforce(float(xi)), xi
    assert oracle.round_to(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 0x3F80   # tie -> even
    assert oracle.round_to(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 0x3F82


# ---------------------------------------------------------------- acceptance helpers

def test_compare_exact_and_normwise():
    ref = np.array([[1.0, -2.0], [3.0, 4.5]])
    ok, _ = compare.check(ref.astype(np.float32), ref, "f32", exact=True)
    assert ok
    bad = ref.astype(np.float32).copy()
    bad.view(np.uint32)[0, 0] += 1           # one ulp
    ok, info = compare.check(bad, ref, "f32", exact=True)
    assert not ok and info["mismatches"] == 1
    ok, info = compare.check(bad, ref, "f32", exact=False)
    assert ok and info["normwise_err"] < 1e-7
    bf = oracle.round_to(ref, "bf16")
    assert compare.check(bf, ref, "bf16", exact=True)[0]
    nan = ref.astype(np.float32).copy()
    nan[1, 1] = np.nan
    assert not compare.check(nan, ref, "f32", exact=False)[0]


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes():
    """Each plausible mistake, planted on the oracle side on the CPU, makes a
    pin above fail: a transposed operand, a wrong storage major, a dropped k
    term, a wrong sign."""
    rng = np.random.Generator(np.random.PCG64(29))
    M, N, K = 4, 3, 5
    a = rng.integers(-5, 6, size=(M, K)).astype(np.float32)
    b = rng.integers(-5, 6, size=(N, K)).astype(np.float32)
    want = np.array([[sum(int(a[m, k]) * int(b[n, k]) for k in range(K)) for n in range(N)]
                     for m in range(M)], dtype=np.float64)
    assert np.array_equal(_oracle_logical(a, b), want)
    # storage read with the wrong major: a square A stored m-major, read as
    # k-major (same buffer size, so both readings stay in bounds)
    sqa = rng.integers(-5, 6, size=(K, K)).astype(np.float32)
    ld = gi.min_ld(K, 4)
    A = gi.store(sqa, True, ld)
    B = gi.store(b, False, ld)
    right = oracle.gemm_ref(K, N, K, "m", "k", "f32", A, ld, B, ld)
    wrong = oracle.gemm_ref(K, N, K, "k", "k", "f32", A, ld, B, ld)
    assert np.array_equal(right, sqa.astype(np.float64) @ b.astype(np.float64).T)
    assert not np.array_equal(wrong, right)
    # dropped last k term
    dropped = _oracle_logical(a[:, :K - 1], b[:, :K - 1])
    assert not np.array_equal(dropped, want)
    # wrong sign on B
    assert not np.array_equal(_oracle_logical(a, -b), want)
    # B used as K x N instead of N x K (only meaningful when shapes allow)
    sq = rng.integers(-5, 6, size=(K, K)).astype(np.float32)
    good = _oracle_logical(a, sq)
    trans = _oracle_logical(a, np.ascontiguousarray(sq.T))
    assert not np.array_equal(good, trans)


# ---------------------------------------------------------------- inputs module

def test_inputs_store_load_roundtrip_and_ranges():
    a, b = gi.draw_ab(300, 200, 100, "int5", seed=1)
    assert a.min() == -5 and a.max() == 5 and np.all(a == np.round(a))
    for first in (False, True):
        ld = (300 if first else 100) + 12
        buf = gi.store(a, first, ld, fill=np.float32(np.nan))
        assert np.array_equal(gi.load(buf, 300, 100, first, ld), a)
        assert np.isnan(buf).sum() == 12 * (100 if first else 300)
    x = np.array([[1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5]], np.float32)
    assert gi.cast(x, "bf16").tolist() == [[0x3F80, 0x3F80, 0x3F82, 0xC020]]


# ---------------------------------------------------------------- epilogue

def test_epilogue_hand_worked_example():
    """alpha, beta and a per-column bias on a 2 x 3 example computed by hand:
    a swapped alpha/beta, a bias along rows, or a dropped term all fail."""
    acc = np.array([[1.0, -2.0, 3.0], [4.0, 5.0, -6.0]])
    c_old = np.array([[10.0, 20.0, 30.0], [40.0, 50.0, 60.0]])
    bias = np.array([0.5, -1.0, 2.0])
    y = oracle.epilogue_ref(acc, alpha=2.0, beta=-0.5, c_old=c_old, bias=bias)
    # row 0: 2 - 5 + 0.5, -4 - 10 - 1, 6 - 15 + 2;  row 1: 8 - 20 + 0.5, 10 - 25 - 1, -12 - 30 + 2
    assert np.array_equal(y, np.array([[-2.5, -15.0, -7.0], [-11.5, -16.0, -40.0]]))
    # beta == 0 never reads C (NaN there does not matter); identity by default
    nan_c = np.full_like(c_old, np.nan)
    assert np.array_equal(oracle.epilogue_ref(acc, c_old=nan_c), acc)
    relu = oracle.epilogue_ref(y, activation=oracle.ACT_RELU)
    assert np.array_equal(relu, np.zeros_like(y))
    assert np.array_equal(oracle.epilogue_ref(acc, activation=oracle.ACT_RELU),
                          np.array([[1.0, 0.0, 3.0], [4.0, 5.0, 0.0]]))


def test_epilogue_relu_special_values():
    x = np.array([[np.nan, -0.0, 0.0, -1e-300, np.inf, -np.inf]])
    y = oracle.epilogue_ref(x, activation=oracle.ACT_RELU)
    assert np.isnan(y[0, 0])
    assert np.signbit(y[0, 1]) and y[0, 1] == 0.0          # -0 is not < 0: kept
    assert y[0, 2] == 0.0 and y[0, 3] == 0.0 and y[0, 4] == np.inf and y[0, 5] == 0.0


def test_epilogue_gelu_closed_forms():
    """gelu(x) = x * Phi(x) with Phi the standard normal CDF: Phi(0) = 1/2,
    Phi(1) = 0.8413447460685429 and Phi(-x) = 1 - Phi(x) (published values of
    the normal distribution), Phi(10) = 1 to double precision."""
    phi1 = 0.8413447460685429
    x = np.array([[0.0, 1.0, -1.0, 2.0, 10.0, -10.0]])
    y = oracle.epilogue_ref(x, activation=oracle.ACT_GELU)[0]
    assert y[0] == 0.0
    assert abs(y[1] - phi1) < 1e-15
    assert abs(y[2] + (1.0 - phi1)) < 1e-15
    assert abs(y[3] - 2.0 * 0.9772498680518208) < 1e-15       # Phi(2)
    assert y[4] == 10.0
    assert -1e-21 <= y[5] <= 0.0          # true value -7.6e-23; 1 + erf(-7.07) rounds to 0
