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
_LIB = os.path.join(_HERE, "liboracle.so")

# Plain C, no fast-math, no FMA contraction: every product of two fp32 or bf16
# values is exact in double, and each sum is left in ascending k.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Werror"]


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc.  Returns the path."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
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
