"""Pins of the CPU oracle (oracle/oracle.c) to facts outside itself.

Each pin is written as a function of an oracle build so that the same pins
also run against deliberately broken copies of oracle.c (the mutation test at
the bottom): a plausible slip in the oracle - a dropped term, a wrong sign, a
transposed operand, a product rounded to FP32 - must fail at least one pin.

Pins:
  * worked examples printed on the pages (tests/golden/*.txt, cited there);
  * exact rational brute force (Python Fractions) on the exactly-summing
    "eighths" inputs of the tutorial "分块计算与矩阵乘法" (section 3) and on random
    dyadic inputs: double sums of such terms are exact, so C and S must match
    the rationals exactly;
  * random FP32 inputs against exact rationals within the textbook bound for
    recursive summation, |fl(sum) - sum| <= (N-1) u / (1 - (N-1) u) * S,
    u = 2**-53;
  * numpy's float64 matrix product as a library routine;
  * algebraic identities: identity matrix, one-hot selection, zero, transpose
    (C^T = B^T A^T, bitwise, since every term and its order are the same),
    N = 1 (a single product, exact in double).
"""

import os
import shutil
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import GOLDEN_FILES, ROOT, load_golden
from synth import eighths_a, eighths_b

U = 2.0**-53


class PinFailure(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _exact(A, B):
    """Rational C and S by the definition, element by element."""
    M, N = A.shape
    K = B.shape[1]
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    C = [[sum((Af[m][n] * Bf[n][k] for n in range(N)), Fraction(0)) for k in range(K)] for m in range(M)]
    S = [[sum((abs(Af[m][n]) * abs(Bf[n][k]) for n in range(N)), Fraction(0)) for k in range(K)] for m in range(M)]
    return C, S


def _dyadic(rng, M, N, K, denom=8, lo=-9, hi=9):
    A = (rng.integers(lo, hi + 1, size=(M, N)) / denom).astype(np.float32)
    B = (rng.integers(lo, hi + 1, size=(N, K)) / denom).astype(np.float32)
    return A, B


# ---------------------------------------------------------------- pins


def pin_worked_examples(orc):
    for name in GOLDEN_FILES:
        M, N, K, A, B, C_expected = load_golden(name)
        C, S = orc.gemm(A, B)
        _check(C.shape == (M, K), f"{name}: shape {C.shape}")
        _check(np.array_equal(C, C_expected), f"{name}: got {C.tolist()} expected {C_expected.tolist()}")
        Ce, _ = orc.gemm_at(A, B, np.repeat(np.arange(M), K), np.tile(np.arange(K), M))
        _check(np.array_equal(Ce.reshape(M, K), C_expected), f"{name}: gemm_at differs")


EXACT_SHAPES = [(1, 1, 1), (2, 3, 2), (3, 5, 4), (4, 7, 5), (17, 19, 23), (6, 31, 9)]


def pin_rational_eighths(orc):
    for (M, N, K) in EXACT_SHAPES:
        A = eighths_a(M * N).reshape(M, N)
        B = eighths_b(N * K).reshape(N, K)
        Cx, Sx = _exact(A, B)
        C, S = orc.gemm(A, B)
        for m in range(M):
            for k in range(K):
                _check(Fraction(C[m, k]) == Cx[m][k], f"eighths {M,N,K} C[{m},{k}] {C[m,k]} != {float(Cx[m][k])}")
                _check(Fraction(S[m, k]) == Sx[m][k], f"eighths {M,N,K} S[{m},{k}] {S[m,k]} != {float(Sx[m][k])}")


def pin_rational_dyadic(orc):
    rng = np.random.default_rng(1234)
    for (M, N, K) in [(3, 4, 5), (5, 3, 2), (8, 16, 7), (2, 33, 3)]:
        A, B = _dyadic(rng, M, N, K)
        Cx, Sx = _exact(A, B)
        C, S = orc.gemm(A, B)
        rows = rng.integers(0, M, size=7)
        cols = rng.integers(0, K, size=7)
        Ca, Sa = orc.gemm_at(A, B, rows, cols)
        for m in range(M):
            for k in range(K):
                _check(Fraction(C[m, k]) == Cx[m][k], f"dyadic {M,N,K} C[{m},{k}]")
                _check(Fraction(S[m, k]) == Sx[m][k], f"dyadic {M,N,K} S[{m},{k}]")
        for i, (m, k) in enumerate(zip(rows, cols)):
            _check(Fraction(Ca[i]) == Cx[m][k], f"dyadic gemm_at C[{m},{k}]")
            _check(Fraction(Sa[i]) == Sx[m][k], f"dyadic gemm_at S[{m},{k}]")


def pin_rational_float_bound(orc):
    rng = np.random.default_rng(99)
    for (M, N, K) in [(4, 40, 3), (3, 97, 4)]:
        A = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(N, K)).astype(np.float32)
        Cx, Sx = _exact(A, B)
        C, S = orc.gemm(A, B)
        g = (N - 1) * U / (1 - (N - 1) * U)
        for m in range(M):
            for k in range(K):
                err = abs(Fraction(C[m, k]) - Cx[m][k])
                _check(err <= Fraction(g) * Sx[m][k], f"float {M,N,K} C[{m},{k}] err {float(err)}")
                # S sums non-negative terms: relative error within the same bound
                errs = abs(Fraction(S[m, k]) - Sx[m][k])
                _check(errs <= Fraction(g) * Sx[m][k], f"float {M,N,K} S[{m},{k}]")
        rows = np.array([0, M - 1, M // 2])
        cols = np.array([K - 1, 0, K // 2])
        Ca, _ = orc.gemm_at(A, B, rows, cols)
        for i, (m, k) in enumerate(zip(rows, cols)):
            _check(abs(Fraction(Ca[i]) - Cx[m][k]) <= Fraction(g) * Sx[m][k], f"float gemm_at C[{m},{k}]")


def pin_numpy_float64(orc):
    rng = np.random.default_rng(7)
    for (M, N, K) in [(1, 1, 1), (1, 300, 5), (7, 129, 33), (64, 64, 64), (33, 5, 70)]:
        A = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
        B = rng.standard_normal(size=(N, K)).astype(np.float32)
        C, S = orc.gemm(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        sref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        bound = 2 * N * U * sref + 1e-300
        _check(np.all(np.abs(C - ref) <= bound), f"numpy {M,N,K}: C max err {np.max(np.abs(C - ref))}")
        _check(np.all(np.abs(S - sref) <= bound), f"numpy {M,N,K}: S max err {np.max(np.abs(S - sref))}")


def pin_identities(orc):
    rng = np.random.default_rng(5)
    # A = I picks B; B = I picks A
    B = rng.uniform(-1, 1, size=(6, 9)).astype(np.float32)
    C, _ = orc.gemm(np.eye(6, dtype=np.float32), B)
    _check(np.array_equal(C, B.astype(np.float64)), "I x B != B")
    A = rng.uniform(-1, 1, size=(5, 6)).astype(np.float32)
    C, _ = orc.gemm(A, np.eye(6, dtype=np.float32))
    _check(np.array_equal(C, A.astype(np.float64)), "A x I != A")
    # one-hot: A[i, j] = 1 copies row j of B into row i, other rows zero
    A = np.zeros((4, 6), dtype=np.float32)
    A[2, 5] = 1.0
    C, _ = orc.gemm(A, B)
    exp = np.zeros((4, 9))
    exp[2] = B[5]
    _check(np.array_equal(C, exp), "one-hot selection")
    # zero
    C, S = orc.gemm(np.zeros((3, 6), dtype=np.float32), B)
    _check(not C.any() and not S.any(), "zero A")
    # transpose: (A B)^T = B^T A^T with the same products in the same order
    A = rng.uniform(-1, 1, size=(7, 11)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(11, 4)).astype(np.float32)
    C, S = orc.gemm(A, B)
    Ct, St = orc.gemm(B.T.copy(), A.T.copy())
    _check(np.array_equal(C.T, Ct) and np.array_equal(S.T, St), "transpose identity")
    # N = 1: outer product, each element one exact product
    a = rng.uniform(-1, 1, size=(5, 1)).astype(np.float32)
    b = rng.uniform(-1, 1, size=(1, 3)).astype(np.float32)
    C, _ = orc.gemm(a, b)
    _check(np.array_equal(C, a.astype(np.float64) * b.astype(np.float64)), "N = 1 outer product")


PINS = [
    pin_worked_examples,
    pin_rational_eighths,
    pin_rational_dyadic,
    pin_rational_float_bound,
    pin_numpy_float64,
    pin_identities,
]


def run_pins(orc):
    failures = []
    for pin in PINS:
        try:
            pin(orc)
        except PinFailure as e:
            failures.append(f"{pin.__name__}: {e}")
    return failures


# ---------------------------------------------------------------- tests


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle(oracle.build())


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_thread_count_does_not_change_bits(orc):
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, size=(37, 50)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(50, 29)).astype(np.float32)
    C1, S1 = orc.gemm(A, B, threads=1)
    C4, S4 = orc.gemm(A, B, threads=4)
    assert np.array_equal(C1, C4) and np.array_equal(S1, S4)


def test_gemm_at_agrees_with_full(orc):
    rng = np.random.default_rng(11)
    A = rng.uniform(-1, 1, size=(19, 23)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(23, 31)).astype(np.float32)
    C, S = orc.gemm(A, B)
    rows = rng.integers(0, 19, size=50)
    cols = rng.integers(0, 31, size=50)
    Ca, Sa = orc.gemm_at(A, B, rows, cols)
    # same terms, same order: bitwise equal
    assert np.array_equal(Ca, C[rows, cols]) and np.array_equal(Sa, S[rows, cols])


def test_gemm_at_rejects_out_of_range(orc):
    A = np.ones((2, 3), dtype=np.float32)
    B = np.ones((3, 4), dtype=np.float32)
    with pytest.raises(IndexError):
        orc.gemm_at(A, B, [2], [0])
    with pytest.raises(IndexError):
        orc.gemm_at(A, B, [0], [4])


def test_shape_mismatch_raises(orc):
    with pytest.raises(ValueError):
        orc.gemm(np.ones((2, 3), np.float32), np.ones((4, 2), np.float32))


def test_tolerance_formula():
    assert oracle.tolerance(0.0) == pytest.approx(1e-6)
    assert oracle.tolerance(2.0) == pytest.approx(2e-5 + 1e-6)


# Each mutant: (label, text in oracle.c, replacement, which occurrence).
MUTANTS = [
    ("full: drop last term", "for (int64_t n = 0; n < N; ++n) {", "for (int64_t n = 0; n + 1 < N; ++n) {", 0),
    ("full: drop first term", "for (int64_t n = 0; n < N; ++n) {", "for (int64_t n = 1; n < N; ++n) {", 0),
    ("full: wrong sign", "c[k] += a * (double)b[k];", "c[k] -= a * (double)b[k];", 0),
    ("full: reversed columns of B", "c[k] += a * (double)b[k];", "c[k] += a * (double)b[K - 1 - k];", 0),
    ("full: product rounded to FP32", "c[k] += a * (double)b[k];", "c[k] += (float)(a * (double)b[k]);", 0),
    ("full: transposed A index", "const double a = (double)A[m * N + n];", "const double a = (double)A[n * M + m];", 0),
    ("full: S without abs", "s[k] += abs_a * fabs((double)b[k]);", "s[k] += a * (double)b[k];", 0),
    ("at: drop last term", "for (int64_t n = 0; n < N; ++n) {", "for (int64_t n = 0; n + 1 < N; ++n) {", 1),
    ("at: transposed B index", "const double b = (double)B[n * K + k];", "const double b = (double)B[k * N + n];", 0),
    ("at: transposed A index", "const double a = (double)A[m * N + n];", "const double a = (double)A[n * M + m];", 1),
]


def _replace_nth(text, old, new, nth):
    idx = -1
    for _ in range(nth + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
@pytest.mark.parametrize("label,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(label, old, new, nth):
    src = open(os.path.join(ROOT, "oracle", "oracle.c"), encoding="utf-8").read()
    assert src.count(old) > nth, f"mutation site for {label!r} not found"
    mutated = _replace_nth(src, old, new, nth)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w", encoding="utf-8") as fh:
            fh.write(mutated)
        lib = oracle.compile_source(path, os.path.join(d, "libmutant.so"))
        failures = run_pins(oracle.Oracle(lib))
    assert failures, f"no pin caught the mutant {label!r}"
