"""Oracle for N-dimensional convolution (1 to 4 spatial dimensions).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``convnd.c``: direct convolution from its definition,
extended to D spatial dimensions the way "Three X's: a new level of working
with large convolutions in PyTorch for model training" extends the 2-D
convolution matrix to 3-D (section "CuBLAS": one more index, one more loop).
This module only marshals numpy arrays.

Shapes: x [batch, C_in, *size], w [C_out, C_in, *kernel], y / dy [batch, C_out, *out].
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from oracle import _load

MAXD = 4


@dataclass(frozen=True)
class NdShape:
    batch: int
    cin: int
    cout: int
    size: tuple
    kernel: tuple
    pad: tuple = None
    stride: tuple = None
    dilation: tuple = None

    def __post_init__(self):
        nd = len(self.size)
        for name, default in (("pad", 0), ("stride", 1), ("dilation", 1)):
            if getattr(self, name) is None:
                object.__setattr__(self, name, (default,) * nd)
        for name in ("size", "kernel", "pad", "stride", "dilation"):
            object.__setattr__(self, name, tuple(int(v) for v in getattr(self, name)))
            if len(getattr(self, name)) != nd:
                raise ValueError("%s must have %d entries" % (name, nd))

    @property
    def nd(self) -> int:
        return len(self.size)

    @property
    def out(self) -> tuple:
        return tuple((s + 2 * p - l * (k - 1) - 1) // t + 1
                     if t >= 1 and l >= 1 and s + 2 * p - l * (k - 1) - 1 >= 0 else 0
                     for s, k, p, t, l in zip(self.size, self.kernel, self.pad, self.stride,
                                              self.dilation))

    @property
    def x_shape(self):
        return (self.batch, self.cin) + self.size

    @property
    def w_shape(self):
        return (self.cout, self.cin) + self.kernel

    @property
    def y_shape(self):
        return (self.batch, self.cout) + self.out

    @property
    def crs(self) -> int:
        return self.cin * int(np.prod(self.kernel))

    @property
    def vol_out(self) -> int:
        return int(np.prod(self.out))

    def packed(self) -> np.ndarray:
        pad4 = lambda v, f: list(v) + [f] * (MAXD - len(v))
        return np.array([self.batch, self.cin, self.cout, self.nd] + pad4(self.size, 1) +
                        pad4(self.kernel, 1) + pad4(self.pad, 0) + pad4(self.stride, 1) +
                        pad4(self.dilation, 1), dtype=np.int64)


_bound = False


def _lib():
    global _bound
    lib = _load()
    if not _bound:
        p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for kind in ("f32", "bf16"):
            for name, args in [("oracle_convnd_fwd_at_", [p, p, p, i64, p, p, p]),
                               ("oracle_convnd_bwd_weight_at_", [p, p, p, i64, p, p, p]),
                               ("oracle_convnd_im2col_", [p, i64, p, p, i64])]:
                fn = getattr(lib, name + kind)
                fn.restype = c_int
                fn.argtypes = args
        _bound = True
    return lib


def _kind(a):
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.uint16:
        return "bf16"
    raise TypeError("float32 or uint16 bf16 bit patterns expected, got %s" % a.dtype)


def _arr(a, shape, kind):
    a = np.ascontiguousarray(a)
    if a.shape != tuple(shape) or _kind(a) != kind:
        raise ValueError("expected %s %s, got %s %s" % (kind, tuple(shape), a.dtype, a.shape))
    return a


def fwd_at(x, w, c: NdShape, flat_idx):
    """y and S at flat output indices (n, co, o...) in row-major order."""
    kind = _kind(x)
    x, w = _arr(x, c.x_shape, kind), _arr(w, c.w_shape, kind)
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64).reshape(-1)
    y, S = np.empty(idx.shape), np.empty(idx.shape)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_convnd_fwd_at_" + kind)(sh.ctypes.data, x.ctypes.data,
                                                         w.ctypes.data, idx.size, idx.ctypes.data,
                                                         y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle convnd fwd: status %d" % rc)
    return y, S


def bwd_weight_at(x, dy, c: NdShape, flat_idx):
    """dw and S at flat filter indices (co, ci, k...) in row-major order."""
    kind = _kind(x)
    x, dy = _arr(x, c.x_shape, kind), _arr(dy, c.y_shape, kind)
    idx = np.ascontiguousarray(flat_idx, dtype=np.int64).reshape(-1)
    dw, S = np.empty(idx.shape), np.empty(idx.shape)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_convnd_bwd_weight_at_" + kind)(
        sh.ctypes.data, x.ctypes.data, dy.ctypes.data, idx.size, idx.ctypes.data, dw.ctypes.data,
        S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle convnd bwd_weight: status %d" % rc)
    return dw, S


def fwd(x, w, c: NdShape):
    """(y, S), full tensors."""
    y, S = fwd_at(x, w, c, np.arange(int(np.prod(c.y_shape))))
    return y.reshape(c.y_shape), S.reshape(c.y_shape)


def bwd_weight(x, dy, c: NdShape):
    """(dw, S), full tensors."""
    dw, S = bwd_weight_at(x, dy, c, np.arange(int(np.prod(c.w_shape))))
    return dw.reshape(c.w_shape), S.reshape(c.w_shape)


def im2col(x, c: NdShape, n: int = 0, ld: int | None = None):
    """The convolution matrix of image n: rows (ci, k...), columns (o...)."""
    kind = _kind(x)
    x = _arr(x, c.x_shape, kind)
    ld = c.vol_out if ld is None else ld
    cols = np.zeros((c.crs, ld), dtype=x.dtype)
    sh = c.packed()
    rc = getattr(_lib(), "oracle_convnd_im2col_" + kind)(sh.ctypes.data, n, x.ctypes.data,
                                                         cols.ctypes.data, ld)
    if rc != 0:
        raise ValueError("oracle convnd im2col: status %d" % rc)
    return cols
