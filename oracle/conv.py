"""Oracle for 2-D convolution: the CPU reference the convolution path is checked
against.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``conv.c``: direct convolution written from its
definition ("Three X's: a new level of working with large convolutions in
PyTorch for model training", sections "Where large convolution kernels come
from" and "CuBLAS"), channel-first tensors, stride, zero padding and dilation,
no filter flip, fp64 sums.  This module only marshals numpy arrays.

Shapes:  x [batch, C_in, H, W],  w [C_out, C_in, R, S],  y / dy [batch, C_out, P, Q].
"""
from __future__ import annotations

import ctypes
from dataclasses import astuple, dataclass

import numpy as np

from oracle import _load, default_threads


@dataclass(frozen=True)
class ConvShape:
    batch: int
    cin: int
    h: int
    w: int
    cout: int
    r: int
    s: int
    ph: int = 0
    pw: int = 0
    sh: int = 1
    sw: int = 1
    dh: int = 1
    dw: int = 1

    @property
    def p(self) -> int:
        return out_dim(self.h, self.ph, self.r, self.sh, self.dh)

    @property
    def q(self) -> int:
        return out_dim(self.w, self.pw, self.s, self.sw, self.dw)

    @property
    def x_shape(self):
        return (self.batch, self.cin, self.h, self.w)

    @property
    def w_shape(self):
        return (self.cout, self.cin, self.r, self.s)

    @property
    def y_shape(self):
        return (self.batch, self.cout, self.p, self.q)

    @property
    def crs(self) -> int:
        return self.cin * self.r * self.s

    def packed(self) -> np.ndarray:
        return np.array(astuple(self), dtype=np.int64)


_i64, _p, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
_bound = False


def _lib():
    global _bound
    lib = _load()
    if not _bound:
        for kind in ("f32", "bf16"):
            for name, args in [
                ("oracle_conv2d_fwd_", [_p, _p, _p, _p, _p, _int]),
                ("oracle_conv2d_bwd_weight_", [_p, _p, _p, _p, _p, _int]),
                ("oracle_conv2d_fwd_entries_", [_p, _p, _p, _i64, _p, _p, _p, _p, _p, _p]),
                ("oracle_conv2d_bwd_weight_entries_", [_p, _p, _p, _i64, _p, _p, _p, _p, _p, _p]),
                ("oracle_im2col_", [_p, _i64, _p, _p, _i64]),
            ]:
                fn = getattr(lib, name + kind)
                fn.restype = _int
                fn.argtypes = args
        lib.oracle_conv_out_dim.restype = _i64
        lib.oracle_conv_out_dim.argtypes = [_i64] * 5
        _bound = True
    return lib


def out_dim(size: int, pad: int, k: int, stride: int, dil: int) -> int:
    """Output extent along one axis: floor((size + 2 pad - dil (k-1) - 1) / stride) + 1,
    0 when the dilated filter does not fit."""
    return int(_lib().oracle_conv_out_dim(size, pad, k, stride, dil))


def _kind(a: np.ndarray) -> str:
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.uint16:
        return "bf16"
    raise TypeError("operands must be float32 or uint16 bf16 bit patterns, got %s" % a.dtype)


def _c(a: np.ndarray, shape, kind: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    if _kind(a) != kind:
        raise TypeError("operands of mixed types")
    return a


def conv2d_fwd(x: np.ndarray, w: np.ndarray, c: ConvShape, threads: int | None = None):
    """(y, S) in float64: the forward convolution and its tolerance scale."""
    kind = _kind(x)
    x, w = _c(x, c.x_shape, kind), _c(w, c.w_shape, kind)
    y = np.empty(c.y_shape, dtype=np.float64)
    S = np.empty(c.y_shape, dtype=np.float64)
    sh = c.packed()
    fn = getattr(_lib(), "oracle_conv2d_fwd_" + kind)
    rc = fn(sh.ctypes.data, x.ctypes.data, w.ctypes.data, y.ctypes.data, S.ctypes.data,
            threads or default_threads())
    if rc != 0:
        raise ValueError("oracle conv2d_fwd: status %d" % rc)
    return y, S


def conv2d_bwd_weight(x: np.ndarray, dy: np.ndarray, c: ConvShape, threads: int | None = None):
    """(dw, S) in float64: the filter gradient and its tolerance scale."""
    kind = _kind(x)
    x, dy = _c(x, c.x_shape, kind), _c(dy, c.y_shape, kind)
    dw = np.empty(c.w_shape, dtype=np.float64)
    S = np.empty(c.w_shape, dtype=np.float64)
    sh = c.packed()
    fn = getattr(_lib(), "oracle_conv2d_bwd_weight_" + kind)
    rc = fn(sh.ctypes.data, x.ctypes.data, dy.ctypes.data, dw.ctypes.data, S.ctypes.data,
            threads or default_threads())
    if rc != 0:
        raise ValueError("oracle conv2d_bwd_weight: status %d" % rc)
    return dw, S


def _idx(*arrays):
    out = [np.ascontiguousarray(a, dtype=np.int64) for a in arrays]
    if len({a.shape for a in out}) != 1 or out[0].ndim != 1:
        raise ValueError("index arrays must be 1-D and of equal length")
    return out


def conv2d_fwd_entries(x, w, c: ConvShape, n, co, p, q):
    """y and S at the positions (n[t], co[t], p[t], q[t]), one sum each."""
    kind = _kind(x)
    x, w = _c(x, c.x_shape, kind), _c(w, c.w_shape, kind)
    n, co, p, q = _idx(n, co, p, q)
    y = np.empty(n.shape, dtype=np.float64)
    S = np.empty(n.shape, dtype=np.float64)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_conv2d_fwd_entries_" + kind)(
        sh.ctypes.data, x.ctypes.data, w.ctypes.data, n.size, n.ctypes.data, co.ctypes.data,
        p.ctypes.data, q.ctypes.data, y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle conv2d_fwd_entries: status %d" % rc)
    return y, S


def conv2d_bwd_weight_entries(x, dy, c: ConvShape, co, ci, r, s):
    """dw and S at the taps (co[t], ci[t], r[t], s[t]), one sum each."""
    kind = _kind(x)
    x, dy = _c(x, c.x_shape, kind), _c(dy, c.y_shape, kind)
    co, ci, r, s = _idx(co, ci, r, s)
    dw = np.empty(co.shape, dtype=np.float64)
    S = np.empty(co.shape, dtype=np.float64)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_conv2d_bwd_weight_entries_" + kind)(
        sh.ctypes.data, x.ctypes.data, dy.ctypes.data, co.size, co.ctypes.data, ci.ctypes.data,
        r.ctypes.data, s.ctypes.data, dw.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle conv2d_bwd_weight_entries: status %d" % rc)
    return dw, S


def im2col(x: np.ndarray, c: ConvShape, n: int = 0, ld: int | None = None) -> np.ndarray:
    """The convolution matrix of image n: rows (ci, r, s), columns (p, q), as
    element bits of x's type; shape (C_in R S, ld), columns beyond P Q zero."""
    kind = _kind(x)
    x = _c(x, c.x_shape, kind)
    ld = c.p * c.q if ld is None else ld
    cols = np.zeros((c.crs, ld), dtype=x.dtype)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_im2col_" + kind)(sh.ctypes.data, n, x.ctypes.data,
                                                  cols.ctypes.data, ld)
    if rc != 0:
        raise ValueError("oracle im2col: status %d" % rc)
    return cols
