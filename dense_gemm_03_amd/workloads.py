"""Seeded synthetic GEMM workloads: shapes, value distributions and generators.

This module holds no GEMM arithmetic.  It only draws operands, so that the GPU
library and the CPU oracle are fed identical bits.  Both sides may import it.

Shapes and distributions (all row-major, tight leading dimensions):

==========  =====================  ==========================  ======
name        M x N x K              entries                     seed
==========  =====================  ==========================  ======
fp32-256    256 x 256 x 256        fp32 uniform[-1, 1]         101
fp32-4096   4096 x 4096 x 4096     fp32 uniform[-1, 1]         102
fp32-1000   1000 x 1000 x 1000     fp32 uniform[-1, 1]         103
fp32-rag    4097 x 4095 x 4099     fp32 uniform[-1, 1]         104
bf16-8192   8192 x 8192 x 8192     normal(0,1) rounded to bf16 105
im2col      64 x 16384 x 61504     fp32 uniform[-1, 1]         106
tall        65536 x 64 x 1024      fp32 uniform[-1, 1]         107
==========  =====================  ==========================  ======

A is drawn with ``seed`` and B with ``seed + 1000`` from
``numpy.random.default_rng``.

Variants of the generalised product C := alpha op(A) op(B) + beta C (the
GEMM page's section "Generalized matrix multiplication GEMM") reuse those
shapes and distributions; the operands are drawn in their stored shapes (A as
K x M when transposed, B as N x K), and an initial C, needed when beta != 0,
is drawn with ``seed + 2000`` in the output type:

==================  ==========  =====  =====  =====  ==========
name                base        op     alpha  beta   C
==================  ==========  =====  =====  =====  ==========
bf16-8192-nt-bf16c  bf16-8192   A B^T  1      0      bf16
bf16-8192-tn-acc    bf16-8192   A^T B  0.5    1      fp32
fp32-4096-tt-ab     fp32-4096   A^T B^T 1.5   -0.5   fp32
==================  ==========  =====  =====  =====  ==========

Convolutions (``CONV_WORKLOADS``, channel-first; "Three X's: large
convolutions in PyTorch for model training"): x, filters and output gradient
drawn with ``seed``, ``seed + 1000`` and ``seed + 2000``, uniform[-1, 1] (fp32)
or normal(0, 1) rounded to bf16:

==================  =====  ======  ========  =====  ======  ===  ====
name                batch  C_in    H x W     C_out  R x S   pad  seed
==================  =====  ======  ========  =====  ======  ===  ====
conv-64c-31k        1      64      128x128   64     31x31   15   108
conv-64c-31k-bf16   1      64      128x128   64     31x31   15   109
conv-small-batch    4      16      40x36     24     5x3     2    110
==================  =====  ======  ========  =====  ======  ===  ====

Convolutions with more spatial dimensions (``CONVND_WORKLOADS``; the same
page's aim of convolution beyond two dimensions: a 3-D filter over a stack of
frames, a 4-D one over a grid of such stacks), drawn the same way; stride and
dilation 1, padding that keeps the output the size of the input:

=================  =====  ====  =====  =============  ==========  ====
name               batch  C_in  C_out  size           kernel      seed
=================  =====  ====  =====  =============  ==========  ====
conv3d-32c-k7      1      32    32     16x64x64       7x7x7       111
conv3d-32c-k7-bf16 1      32    32     16x64x64       7x7x7       112
conv4d-16c-k5      2      16    32     6x6x24x24      3x3x5x5     113
=================  =====  ====  =====  =============  ==========  ====

Large operands are drawn in row chunks; the
PCG64 stream yields the same values whether drawn at once or in chunks.

The im2col shape is the weight-gradient GEMM of a 2-D convolution with a large
kernel ("Three X's: large convolutions in PyTorch for model training",
sections on where large kernels come from and on the im2col route through
cuBLAS): 64 output channels, 64 input channels times a 31 x 31 kernel area
(K = 61504) and 128 x 128 output positions (N = 16384).  Its operands here are
i.i.d. uniform, without the repeated entries a real column matrix carries.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

_CHUNK_ELEMS = 1 << 24  # draw at most 16M values at a time


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" or "bf16" (bf16 inputs, fp32 output)
    M: int
    N: int
    K: int
    dist: str  # "uniform" or "normal_bf16"
    seed: int
    transa: bool = False
    transb: bool = False
    alpha: float = 1.0
    beta: float = 0.0
    out: str = "f32"  # type of C: "f32" or "bf16"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def out_bytes(self) -> int:
        return 4 if self.out == "f32" else 2

    @property
    def plain(self) -> bool:
        """The plain product C = A . B with fp32 C."""
        return (not self.transa and not self.transb and self.alpha == 1.0 and self.beta == 0.0
                and self.out == "f32")

    @property
    def a_shape(self):
        return (self.K, self.M) if self.transa else (self.M, self.K)

    @property
    def b_shape(self):
        return (self.N, self.K) if self.transb else (self.K, self.N)

    @property
    def algorithmic_bytes(self) -> int:
        """Compulsory HBM bytes: read A and B once, write C once, and read C
        once when beta != 0."""
        c_passes = 2 if self.beta != 0.0 else 1
        return (self.M * self.K + self.K * self.N) * self.in_bytes \
            + c_passes * self.M * self.N * self.out_bytes

    def operands(self):
        """(A, B) in their stored shapes as numpy arrays: float32, or uint16
        bf16 bit patterns."""
        if self.dist == "uniform":
            return (uniform_f32(self.a_shape, self.seed),
                    uniform_f32(self.b_shape, self.seed + 1000))
        if self.dist == "normal_bf16":
            return (normal_bf16_bits(self.a_shape, self.seed),
                    normal_bf16_bits(self.b_shape, self.seed + 1000))
        raise ValueError(self.dist)

    def initial_c(self):
        """The initial C (M x N) for beta != 0: float32 uniform[-1, 1], or
        normal(0, 1) rounded to bf16 bit patterns for bf16 C."""
        if self.out == "f32":
            return uniform_f32((self.M, self.N), self.seed + 2000)
        return normal_bf16_bits((self.M, self.N), self.seed + 2000)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32-256", "f32", 256, 256, 256, "uniform", 101),
        Workload("fp32-4096", "f32", 4096, 4096, 4096, "uniform", 102),
        Workload("fp32-1000", "f32", 1000, 1000, 1000, "uniform", 103),
        Workload("fp32-rag", "f32", 4097, 4095, 4099, "uniform", 104),
        Workload("bf16-8192", "bf16", 8192, 8192, 8192, "normal_bf16", 105),
        Workload("im2col", "f32", 64, 16384, 61504, "uniform", 106),
        Workload("tall", "f32", 65536, 64, 1024, "uniform", 107),
    ]
}

VARIANTS = {
    w.name: w
    for w in [
        Workload("bf16-8192-nt-bf16c", "bf16", 8192, 8192, 8192, "normal_bf16", 105,
                 transb=True, out="bf16"),
        Workload("bf16-8192-tn-acc", "bf16", 8192, 8192, 8192, "normal_bf16", 105,
                 transa=True, alpha=0.5, beta=1.0),
        Workload("fp32-4096-tt-ab", "f32", 4096, 4096, 4096, "uniform", 102,
                 transa=True, transb=True, alpha=1.5, beta=-0.5),
    ]
}


def _rows_per_chunk(cols: int) -> int:
    return max(1, _CHUNK_ELEMS // max(cols, 1))


def _rows_cols(shape):
    """An N-D shape seen as (product of the leading dimensions, last dimension):
    values are drawn row by row of that 2-D view, so a 2-D shape draws exactly
    what it always did."""
    shape = tuple(int(d) for d in shape)
    if len(shape) == 1:
        return 1, shape[0], shape
    return int(np.prod(shape[:-1], dtype=np.int64)), shape[-1], shape


def uniform_f32(shape, seed: int) -> np.ndarray:
    """i.i.d. uniform[-1, 1) float32 values (drawn in float64, then rounded)."""
    rows, cols, shape = _rows_cols(shape)
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), dtype=np.float32)
    step = _rows_per_chunk(cols)
    for r in range(0, rows, step):
        r1 = min(rows, r + step)
        out[r:r1] = rng.uniform(-1.0, 1.0, size=(r1 - r, cols))
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the
    16-bit patterns.  Inputs must be finite (the generators only make finite
    values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def normal_bf16_bits(shape, seed: int) -> np.ndarray:
    """i.i.d. standard normal values, drawn as float32 and rounded to bf16."""
    rows, cols, shape = _rows_cols(shape)
    rng = np.random.default_rng(seed)
    out = np.empty((rows, cols), dtype=np.uint16)
    step = _rows_per_chunk(cols)
    for r in range(0, rows, step):
        r1 = min(rows, r + step)
        out[r:r1] = f32_to_bf16_bits(rng.standard_normal(size=(r1 - r, cols), dtype=np.float32))
    return out.reshape(shape)


def small_int_f32(shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers in [lo, hi] stored as float32.  Every partial sum of products of
    such values is an exact integer well below 2^24, so any summation order
    gives the same bits."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def small_int_bf16_bits(shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers in [lo, hi] as bf16 bit patterns (exactly representable)."""
    return f32_to_bf16_bits(small_int_f32(shape, seed, lo, hi))


def sample_positions(M: int, N: int, count: int, seed: int):
    """``count`` (i, j) positions spread over an M x N output: its four corners,
    the last row and column, and the rest uniform at random."""
    rng = np.random.default_rng(seed)
    fixed_i = [0, 0, M - 1, M - 1]
    fixed_j = [0, N - 1, 0, N - 1]
    extra = max(0, count - len(fixed_i))
    I = np.concatenate([np.array(fixed_i), rng.integers(0, M, size=extra)])
    J = np.concatenate([np.array(fixed_j), rng.integers(0, N, size=extra)])
    return I.astype(np.int64), J.astype(np.int64)


# ------------------------------------------------------------ convolutions --

@dataclass(frozen=True)
class ConvWorkload:
    """A 2-D convolution, channel-first: x (batch, cin, h, w), filters
    (cout, cin, r, s), output (batch, cout, p, q)."""
    name: str
    dtype: str  # "f32" or "bf16" (x, w and dy)
    batch: int
    cin: int
    h: int
    w: int
    cout: int
    r: int
    s: int
    pad: int
    stride: int
    dilation: int
    seed: int

    @property
    def p(self) -> int:
        return (self.h + 2 * self.pad - self.dilation * (self.r - 1) - 1) // self.stride + 1

    @property
    def q(self) -> int:
        return (self.w + 2 * self.pad - self.dilation * (self.s - 1) - 1) // self.stride + 1

    @property
    def crs(self) -> int:
        return self.cin * self.r * self.s

    @property
    def flops(self) -> int:
        """Multiply-adds of the forward pass (or of the filter gradient) x 2."""
        return 2 * self.batch * self.cout * self.p * self.q * self.crs

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def im2col_bytes(self) -> int:
        """Compulsory HBM bytes of one image's convolution matrix: read the
        image once, write the matrix once."""
        return (self.cin * self.h * self.w + self.crs * self.p * self.q) * self.in_bytes

    def _draw(self, shape, seed):
        if self.dtype == "f32":
            return uniform_f32(shape, seed)
        return normal_bf16_bits(shape, seed)

    def x(self):
        return self._draw((self.batch, self.cin, self.h, self.w), self.seed)

    def weights(self):
        return self._draw((self.cout, self.cin, self.r, self.s), self.seed + 1000)

    def dy(self):
        return self._draw((self.batch, self.cout, self.p, self.q), self.seed + 2000)


# The large-kernel convolution whose forward GEMM is the im2col workload above
# (64 x 16384 x 61504): 64 channels in and out, 31 x 31 filters, 128 x 128
# images with "same" zero padding.  Its filter gradient is the GEMM
# 64 x 61504 x 16384 with the convolution matrix transposed.
CONV_WORKLOADS = {
    c.name: c
    for c in [
        ConvWorkload("conv-64c-31k", "f32", 1, 64, 128, 128, 64, 31, 31, 15, 1, 1, 108),
        ConvWorkload("conv-64c-31k-bf16", "bf16", 1, 64, 128, 128, 64, 31, 31, 15, 1, 1, 109),
        ConvWorkload("conv-small-batch", "f32", 4, 16, 40, 36, 24, 5, 3, 2, 1, 1, 110),
    ]
}


@dataclass(frozen=True)
class ConvNdWorkload:
    """A convolution with len(size) spatial dimensions, channel-first:
    x (batch, cin, *size), filters (cout, cin, *kernel), output (batch, cout,
    *out); stride and dilation 1, padding pad per dimension."""
    name: str
    dtype: str  # "f32" or "bf16" (x, w and dy)
    batch: int
    cin: int
    cout: int
    size: tuple
    kernel: tuple
    pad: tuple
    seed: int

    @property
    def nd(self) -> int:
        return len(self.size)

    @property
    def stride(self) -> tuple:
        return (1,) * self.nd

    @property
    def dilation(self) -> tuple:
        return (1,) * self.nd

    @property
    def out(self) -> tuple:
        return tuple(s + 2 * p - k + 1 for s, k, p in zip(self.size, self.kernel, self.pad))

    @property
    def vol_out(self) -> int:
        return int(np.prod(self.out))

    @property
    def crs(self) -> int:
        return self.cin * int(np.prod(self.kernel))

    @property
    def flops(self) -> int:
        """Multiply-adds of the forward pass (or of the filter gradient) x 2."""
        return 2 * self.batch * self.cout * self.vol_out * self.crs

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def im2col_bytes(self) -> int:
        """Compulsory HBM bytes of one image's convolution matrix: read the
        image once, write the matrix once."""
        return (self.cin * int(np.prod(self.size)) + self.crs * self.vol_out) * self.in_bytes

    def _draw(self, shape, seed):
        if self.dtype == "f32":
            return uniform_f32(shape, seed)
        return normal_bf16_bits(shape, seed)

    def x(self):
        return self._draw((self.batch, self.cin) + tuple(self.size), self.seed)

    def weights(self):
        return self._draw((self.cout, self.cin) + tuple(self.kernel), self.seed + 1000)

    def dy(self):
        return self._draw((self.batch, self.cout) + self.out, self.seed + 2000)


# A 7 x 7 x 7 filter over 16 frames of 64 x 64 (convolution matrix 10976 x
# 65536: 2.9 GB in fp32) and a 3 x 3 x 5 x 5 filter over a 6 x 6 grid of
# 24 x 24 images.
CONVND_WORKLOADS = {
    c.name: c
    for c in [
        ConvNdWorkload("conv3d-32c-k7", "f32", 1, 32, 32, (16, 64, 64), (7, 7, 7), (3, 3, 3), 111),
        ConvNdWorkload("conv3d-32c-k7-bf16", "bf16", 1, 32, 32, (16, 64, 64), (7, 7, 7),
                       (3, 3, 3), 112),
        ConvNdWorkload("conv4d-16c-k5", "f32", 2, 16, 32, (6, 6, 24, 24), (3, 3, 5, 5),
                       (1, 1, 2, 2), 113),
    ]
}
