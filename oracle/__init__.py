"""Oracle for dense GEMM: the CPU reference that the GPU library is checked against.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, ascending k):
the definition of the matrix product from "Learning to develop for GPUs through
the GEMM operation", section "Matrix product" -- C[i][j] is the sum over k of
A[i][k] * B[k][j] -- written for row-major storage with leading dimensions.
Alongside C it returns S[i][j] = sum_k |A[i][k]| * |B[k][j]|, the scale of the
tolerance test |C - C_ref| <= tol * S.

This module only marshals numpy arrays into that C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SOURCES = [_SRC, os.path.join(_HERE, "conv.c"), os.path.join(_HERE, "convnd.c")]
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain C, no fast-math, no FMA contraction: every product of two fp32 or bf16
# values is exact in double, and each sum is left in ascending k.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Werror"]


def build() -> str:
    """Compile ``oracle.c``, ``conv.c`` and ``convnd.c`` into ``liboracle.so`` with gcc.
    Returns the path."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, *_SOURCES, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(src)
                                       for src in _SOURCES):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    for name in ("oracle_gemm_f32", "oracle_gemm_bf16"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, i64, ctypes.c_int]
    for name in ("oracle_entries_f32", "oracle_entries_bf16"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, i64, p, p, p, p]
    _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover - non-Linux
        return max(1, os.cpu_count() or 1)


def _operand(x: np.ndarray, dtype) -> tuple[np.ndarray, int]:
    """Check a 2-D operand with unit column stride; return it and its leading dim."""
    if x.ndim != 2 or x.dtype != dtype:
        raise TypeError("expected a 2-D %s array, got %s %s" % (np.dtype(dtype), x.dtype, x.shape))
    if x.size == 0:
        return x, max(x.shape[1], 1)
    if x.shape[1] > 1 and x.strides[1] != x.itemsize:
        raise ValueError("operand rows must be contiguous")
    ld = x.strides[0] // x.itemsize if x.shape[0] > 1 else max(x.shape[1], 1)
    return x, max(int(ld), max(x.shape[1], 1))


def _gemm(kind: str, A: np.ndarray, B: np.ndarray, threads: int | None, with_s: bool):
    dtype = np.float32 if kind == "f32" else np.uint16
    A, lda = _operand(A, dtype)
    B, ldb = _operand(B, dtype)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: A is %s, B is %s" % (A.shape, B.shape))
    C = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64) if with_s else None
    lib = _load()
    fn = lib.oracle_gemm_f32 if kind == "f32" else lib.oracle_gemm_bf16
    rc = fn(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
            C.ctypes.data, max(N, 1), S.ctypes.data if S is not None else None, max(N, 1),
            threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle returned status %d" % rc)
    return (C, S) if with_s else C


def gemm_f32(A: np.ndarray, B: np.ndarray, threads: int | None = None, with_s: bool = True):
    """C_ref (and S) in float64 for fp32 operands A (M x K) and B (K x N)."""
    return _gemm("f32", A, B, threads, with_s)


def gemm_bf16(A_bits: np.ndarray, B_bits: np.ndarray, threads: int | None = None,
              with_s: bool = True):
    """C_ref (and S) in float64 for bf16 operands given as uint16 bit patterns."""
    return _gemm("bf16", A_bits, B_bits, threads, with_s)


def _entries(kind: str, A, B, I, J):
    dtype = np.float32 if kind == "f32" else np.uint16
    A, lda = _operand(A, dtype)
    B, ldb = _operand(B, dtype)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D and of equal length")
    C = np.empty(I.shape, dtype=np.float64)
    S = np.empty(I.shape, dtype=np.float64)
    lib = _load()
    fn = lib.oracle_entries_f32 if kind == "f32" else lib.oracle_entries_bf16
    rc = fn(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb, I.size,
            I.ctypes.data, J.ctypes.data, C.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle returned status %d" % rc)
    return C, S


def entries_f32(A, B, I, J):
    """C_ref[I[t], J[t]] and S[I[t], J[t]] for fp32 operands, one dot product each."""
    return _entries("f32", A, B, I, J)


def entries_bf16(A_bits, B_bits, I, J):
    """C_ref[I[t], J[t]] and S[I[t], J[t]] for bf16 operands (uint16 bit patterns)."""
    return _entries("bf16", A_bits, B_bits, I, J)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns: the 16 bits are the top half of a binary32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def max_error_ratio(C, C_ref: np.ndarray, S: np.ndarray) -> tuple[float, bool]:
    """Largest |C - C_ref| / S over entries with S > 0, and whether every entry
    with S == 0 holds exactly 0 (an empty or all-zero sum must come out as 0)."""
    C = np.asarray(C, dtype=np.float64)
    err = np.abs(C - C_ref)
    pos = S > 0
    ratio = float(np.max(err[pos] / S[pos])) if np.any(pos) else 0.0
    if not np.all(np.isfinite(C[pos])):
        ratio = float("inf")
    zeros_ok = bool(np.all(C[~pos] == 0.0))
    return ratio, zeros_ok


def _stored_to_op(X: np.ndarray, trans: bool) -> np.ndarray:
    """op(X): X itself, or a row-major copy of its transpose."""
    return np.ascontiguousarray(X.T) if trans else X


def gemm_general(A: np.ndarray, B: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                 C0: np.ndarray | None = None, transa: bool = False, transb: bool = False,
                 kind: str = "f32", threads: int | None = None):
    """The generalised product of "Learning to develop for GPUs through the GEMM
    operation", section "Generalized matrix multiplication GEMM": the matrix
    product weighted by alpha, plus the accumulator C0 weighted by beta,

        C = alpha * op(A) . op(B) + beta * C0,    op(X) = X or X^T,

    in float64.  A and B are the stored matrices (``kind`` "f32": float32,
    "bf16": uint16 bit patterns): A is M x K, or K x M when ``transa``; B is
    K x N, or N x K when ``transb``.  op() is a transposed copy; the product is
    the C code above.  alpha and beta are applied exactly in float64 to that
    exact product.  C0 is the initial C as float64 (decoded when C is bf16).

    The conventions of the BLAS routine this generalises (a reading, the page's
    formula being an image): C0 is not read when beta == 0 (it may hold NaN),
    and A and B are not read when alpha == 0 or K == 0.

    Returns (C_ref, S) with S = |alpha| * sum_k |op(A)[i][k]| |op(B)[k][j]|
    + |beta| * |C0[i][j]|, the scale of the tolerance test."""
    opA = _stored_to_op(A, transa)
    opB = _stored_to_op(B, transb)
    M, K = opA.shape
    K2, N = opB.shape
    if K != K2:
        raise ValueError("inner dimensions differ: op(A) is %s, op(B) is %s" % (opA.shape, opB.shape))
    alpha = float(alpha)
    beta = float(beta)
    if alpha != 0.0 and K > 0:
        P, SP = _gemm(kind, opA, opB, threads, True)
        C = alpha * P
        S = abs(alpha) * SP
    else:
        C = np.zeros((M, N), dtype=np.float64)
        S = np.zeros((M, N), dtype=np.float64)
    if beta != 0.0:
        if C0 is None or C0.shape != (M, N):
            raise ValueError("beta != 0 needs C0 of shape (%d, %d)" % (M, N))
        C0 = np.asarray(C0, dtype=np.float64)
        C = C + beta * C0
        S = S + abs(beta) * np.abs(C0)
    return C, S


def round_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (8 significant bits), ties to
    the even significand, and return the bit patterns; overflow gives +-inf and
    NaN a quiet NaN.  Subnormals keep the binary32 spacing 2^-133.  The steps,
    applied to every element at once: |v| = m 2^e with 0.5 <= m < 1, so 8-bit
    significands are spaced 2^(e-8) apart (never closer than 2^-133); v is
    rounded to a multiple of that spacing, halves to even; the result is
    exactly representable in binary32, whose upper 16 bits are the bf16."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)
        step = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 8, -133))
        q = np.rint(x / step) * step                  # np.rint rounds halves to even
        q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, x), q)
        q = np.where(np.isinf(x) | (x == 0.0), x, q)  # infinities and signed zeros as they are
        bits = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits.reshape(x.shape)


def entries_general(A: np.ndarray, B: np.ndarray, I, J, alpha: float = 1.0, beta: float = 0.0,
                    C0_at: np.ndarray | None = None, transa: bool = False,
                    transb: bool = False, kind: str = "f32"):
    """gemm_general at the positions (I[t], J[t]) only, one dot product each:
    (C_ref, S) at those positions.  C0_at holds the initial C at the same
    positions (float64; read only when beta != 0).  Same conventions as
    gemm_general."""
    opA = _stored_to_op(A, transa)
    opB = _stored_to_op(B, transb)
    I = np.ascontiguousarray(I, dtype=np.int64)
    alpha = float(alpha)
    beta = float(beta)
    if alpha != 0.0 and opA.shape[1] > 0:
        P, SP = _entries(kind, opA, opB, I, J)
        C, S = alpha * P, abs(alpha) * SP
    else:
        C, S = np.zeros(I.shape), np.zeros(I.shape)
    if beta != 0.0:
        C0_at = np.asarray(C0_at, dtype=np.float64)
        C, S = C + beta * C0_at, S + abs(beta) * np.abs(C0_at)
    return C, S
