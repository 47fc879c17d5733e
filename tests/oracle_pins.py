"""Pins for the oracle: checks that tie it to facts fixed by the mathematics of
the matrix product, not to a second copy of itself.

The definition pinned ("Learning to develop for GPUs through the GEMM
operation", section "Matrix product"): C = A . B with A of size M x K, B of
size K x N, C[i][j] = sum_k A[i][k] * B[k][j]; and the tolerance scale
S[i][j] = sum_k |A[i][k]| * |B[k][j]|.

Each pin takes ``gemm(A, B) -> (C, S)`` over float64-valued numpy arrays (the
caller picks the operand encoding), so the same pins run against the real
oracle and against mutants with planted mistakes, which must each fail at
least one pin.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

from dense_gemm_03_amd.workloads import small_int_f32


class PinFailure(AssertionError):
    pass


def _quant(gemm, x: np.ndarray) -> np.ndarray:
    """Round test values to what the operand encoding under test can hold
    (``gemm.quantize``; float32 if the callable has none)."""
    q = getattr(gemm, "quantize", None)
    return q(x) if q is not None else np.asarray(x, dtype=np.float32).astype(np.float64)


def _check(cond: bool, msg: str):
    if not cond:
        raise PinFailure(msg)


def exact_product(A: np.ndarray, B: np.ndarray):
    """Brute force in exact rational arithmetic (fractions.Fraction): the
    definition term by term, no rounding anywhere."""
    M, K = A.shape
    _, N = B.shape
    Af = [[Fraction(float(A[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B[k, j])) for j in range(N)] for k in range(K)]
    C = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    S = [[sum((abs(Af[i][k]) * abs(Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)]
         for i in range(M)]
    return C, S


def pin_bruteforce_integers(gemm, max_dim=8, seed=7):
    """Every shape (m, n, k) in {1..max_dim}^3 with integer entries in [-3, 3]:
    all sums are exact in fp64, so C and S must equal the rational result."""
    rng = np.random.default_rng(seed)
    for m, n, k in itertools.product(range(1, max_dim + 1), repeat=3):
        A = rng.integers(-3, 4, size=(m, k)).astype(np.float64)
        B = rng.integers(-3, 4, size=(k, n)).astype(np.float64)
        C, S = gemm(A, B)
        Ce, Se = exact_product(A, B)
        _check(C.shape == (m, n), "shape %s for %dx%dx%d" % (C.shape, m, n, k))
        for i in range(m):
            for j in range(n):
                _check(Fraction(float(C[i, j])) == Ce[i][j],
                       "C[%d,%d] of %dx%dx%d: %r vs exact %s" % (i, j, m, n, k, C[i, j], Ce[i][j]))
                _check(Fraction(float(S[i, j])) == Se[i][j],
                       "S[%d,%d] of %dx%dx%d: %r vs exact %s" % (i, j, m, n, k, S[i, j], Se[i][j]))


def pin_bruteforce_reals(gemm, make_value, shapes, seed=11):
    """Random real entries (given encoding): the fp64 sums may round, but each
    must lie within (k-1) * 2^-53 * S of the exact rational sum (the standard
    bound for recursive summation of exact products)."""
    rng = np.random.default_rng(seed)
    u = 2.0 ** -53
    for (m, n, k) in shapes:
        A = make_value(rng, (m, k))
        B = make_value(rng, (k, n))
        C, S = gemm(A, B)
        Ce, Se = exact_product(A, B)
        for i in range(m):
            for j in range(n):
                bound = Fraction(max(k - 1, 0)) * Fraction(u) * Se[i][j] * Fraction(1 + 1e-12)
                _check(abs(Fraction(float(C[i, j])) - Ce[i][j]) <= bound,
                       "C[%d,%d] of %dx%dx%d outside the fp64 summation bound" % (i, j, m, n, k))
                _check(abs(Fraction(float(S[i, j])) - Se[i][j]) <= bound,
                       "S[%d,%d] of %dx%dx%d outside the fp64 summation bound" % (i, j, m, n, k))


def pin_identity(gemm, M=37, N=29, seed=3):
    """A = I (M x M) gives C = B; B = I (N x N) gives C = A, exactly."""
    rng = np.random.default_rng(seed)
    B = _quant(gemm, rng.uniform(-1, 1, size=(M, N)))
    C, S = gemm(np.eye(M), B)
    _check(np.array_equal(C, B), "I . B != B")
    _check(np.array_equal(S, np.abs(B)), "S of I . B != |B|")
    A = _quant(gemm, rng.uniform(-1, 1, size=(M, N)))
    C, _ = gemm(A, np.eye(N))
    _check(np.array_equal(C, A), "A . I != A")


def pin_all_ones(gemm, shapes=((1, 1, 1), (5, 3, 7), (33, 65, 129), (64, 17, 1000))):
    """A = 1 and B = 1 give C[i][j] = K everywhere (and S = K)."""
    for (m, n, k) in shapes:
        C, S = gemm(np.ones((m, k)), np.ones((k, n)))
        _check(np.all(C == k) and np.all(S == k), "all-ones %dx%dx%d: C != K" % (m, n, k))
        # Sign pattern: A = -1, B = 1 gives -K; S stays K.
        C, S = gemm(-np.ones((m, k)), np.ones((k, n)))
        _check(np.all(C == -k) and np.all(S == k), "(-1).(1) %dx%dx%d: C != -K" % (m, n, k))


def pin_diagonal(gemm, M=23, N=31, seed=5):
    """A = diag(d) scales the rows of B: C[i][j] = d_i * B[i][j] (one exact
    product per entry)."""
    rng = np.random.default_rng(seed)
    d = _quant(gemm, rng.uniform(-2, 2, size=M))
    B = _quant(gemm, rng.uniform(-1, 1, size=(M, N)))
    C, _ = gemm(np.diag(d), B)
    _check(np.array_equal(C, d[:, None] * B), "diag(d) . B != d_i * B_ij")
    # and B = diag(e) scales the columns of A
    e = _quant(gemm, rng.uniform(-2, 2, size=N))
    A = _quant(gemm, rng.uniform(-1, 1, size=(M, N)))
    C, _ = gemm(A, np.diag(e))
    _check(np.array_equal(C, A * e[None, :]), "A . diag(e) != A_ij * e_j")


def pin_one_hot(gemm, M=9, N=13, K=11, seed=9):
    """A = e_i e_k^T selects row k of B into row i of C, and nothing else."""
    rng = np.random.default_rng(seed)
    B = rng.integers(-9, 10, size=(K, N)).astype(np.float64)
    for i, k in [(0, 0), (M - 1, K - 1), (3, 7), (8, 2)]:
        A = np.zeros((M, K))
        A[i, k] = 1.0
        C, _ = gemm(A, B)
        want = np.zeros((M, N))
        want[i] = B[k]
        _check(np.array_equal(C, want), "one-hot (%d,%d) misplaced" % (i, k))


def pin_transpose(gemm, M=19, N=27, K=45, seed=13):
    """(A . B)^T = B^T . A^T bitwise: the same products, the same k order."""
    rng = np.random.default_rng(seed)
    A = _quant(gemm, rng.uniform(-1, 1, size=(M, K)))
    B = _quant(gemm, rng.uniform(-1, 1, size=(K, N)))
    C, S = gemm(A, B)
    Ct, St = gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    _check(np.array_equal(C.T, Ct), "(A.B)^T != B^T.A^T")
    _check(np.array_equal(S.T, St), "S(A,B)^T != S(B^T,A^T)")


def pin_small_int_any_shape(gemm, shapes=((130, 70, 300), (1, 257, 513), (257, 1, 65))):
    """Small-integer operands at shapes past any blocking: the result is an
    exact integer matrix, checked against integer matrix multiplication
    (numpy int64 matmul, exact)."""
    for t, (m, n, k) in enumerate(shapes):
        A = small_int_f32((m, k), 100 + t).astype(np.float64)
        B = small_int_f32((k, n), 200 + t).astype(np.float64)
        C, S = gemm(A, B)
        Ai, Bi = A.astype(np.int64), B.astype(np.int64)
        _check(np.array_equal(C, (Ai @ Bi).astype(np.float64)), "integer product %dx%dx%d" % (m, n, k))
        _check(np.array_equal(S, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64)),
               "integer S %dx%dx%d" % (m, n, k))


ALL_PINS = [
    pin_identity,
    pin_all_ones,
    pin_diagonal,
    pin_one_hot,
    pin_transpose,
    pin_small_int_any_shape,
    lambda g: pin_bruteforce_integers(g, max_dim=5),
]
