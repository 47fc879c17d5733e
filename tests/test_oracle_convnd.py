"""The N-dimensional convolution oracle against its pins (CPU only).

``oracle.convnd`` is direct convolution in 1 to 4 spatial dimensions
(channel-first, stride / zero padding / dilation per dimension, no filter
flip) and its filter gradient, extending the 2-D case the way "Three X's:
large convolutions in PyTorch for model training" extends it (section
"CuBLAS": one more index and one more loop per dimension).  Pins:
  * two dimensions equal the pinned 2-D oracle bit for bit (forward, filter
    gradient and convolution matrix);
  * one dimension equals numpy's correlate, exact on integers;
  * three and four dimensions equal scipy's N-D direct correlation of the
    zero-padded image with a zero-stuffed (dilated) filter, subsampled by the
    stride, exact on integers, summed over channels;
  * torch's float64 conv1d / conv3d and their autograd filter gradients, within
    the fp64 summation bound;
  * the adjoint identity <conv(x, w), dy> = <w, dW(x, dy)> in 3-D and 4-D;
  * an all-ones closed form in 4-D;
  * the convolution matrix times the filters equals the direct convolution
    bit for bit.
Mutants with planted mistakes each fail at least one pin.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import conv as oc
from oracle import convnd as ond
from oracle.convnd import NdShape


class PinFailure(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _ints(shape, seed):
    return np.random.default_rng(seed).integers(-3, 4, size=shape).astype(np.float32)


def _scipy_ref(x, w, c: NdShape):
    """Multi-channel reference from scipy's N-D correlation (float64)."""
    out = np.zeros(c.y_shape)
    for n in range(c.batch):
        for co in range(c.cout):
            for ci in range(c.cin):
                xp = np.pad(x[n, ci].astype(np.float64), [(p, p) for p in c.pad])
                wd = np.zeros([(k - 1) * l + 1 for k, l in zip(c.kernel, c.dilation)])
                wd[tuple(slice(None, None, l) for l in c.dilation)] = w[co, ci]
                full = scipy.signal.correlate(xp, wd, mode="valid", method="direct")
                out[n, co] += full[tuple(slice(None, None, t) for t in c.stride)]
    return out


def _real_fwd(x, w, c):
    return ond.fwd(x, w, c)


def _real_bwd(x, dy, c):
    return ond.bwd_weight(x, dy, c)


# ------------------------------------------------------------------- pins --

def pin_two_dims_is_the_2d_oracle(fwd, bwd):
    rng = np.random.default_rng(1)
    for c in [NdShape(2, 3, 4, (9, 8), (3, 2), (1, 1), (2, 1), (1, 2)),
              NdShape(1, 2, 3, (7, 7), (3, 3), (1, 1))]:
        c2 = oc.ConvShape(c.batch, c.cin, c.size[0], c.size[1], c.cout, c.kernel[0], c.kernel[1],
                          c.pad[0], c.pad[1], c.stride[0], c.stride[1], c.dilation[0],
                          c.dilation[1])
        x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
        w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
        dy = rng.uniform(-1, 1, c.y_shape).astype(np.float32)
        y, S = fwd(x, w, c)
        y2, S2 = oc.conv2d_fwd(x, w, c2)
        _check(np.array_equal(y, y2) and np.array_equal(S, S2), "2-D forward differs")
        g, Sg = bwd(x, dy, c)
        g2, Sg2 = oc.conv2d_bwd_weight(x, dy, c2)
        _check(np.array_equal(g, g2) and np.array_equal(Sg, Sg2), "2-D filter gradient differs")


def pin_one_dim_numpy(fwd, bwd):
    for t, (L, K, p, st, dl) in enumerate([(20, 3, 0, 1, 1), (17, 4, 2, 2, 1), (23, 3, 1, 3, 4)]):
        c = NdShape(1, 1, 1, (L,), (K,), (p,), (st,), (dl,))
        x, w = _ints(c.x_shape, 10 + t), _ints(c.w_shape, 20 + t)
        wd = np.zeros((K - 1) * dl + 1)
        wd[::dl] = w[0, 0]
        want = np.correlate(np.pad(x[0, 0].astype(np.float64), p), wd, mode="valid")[::st]
        y, _ = fwd(x, w, c)
        _check(y.shape[2:] == want.shape and np.array_equal(y[0, 0], want), "1-D case %d" % t)


def pin_three_four_dims_scipy(fwd, bwd):
    for t, c in enumerate([
            NdShape(2, 2, 3, (6, 7, 5), (3, 2, 3), (1, 0, 1), (1, 2, 1), (1, 1, 2)),
            NdShape(1, 2, 2, (5, 4, 6, 5), (2, 3, 2, 2), (1, 1, 0, 1), (2, 1, 1, 2), (1, 1, 2, 1)),
            NdShape(1, 1, 1, (4, 4, 4, 4), (3, 3, 3, 3), (1, 1, 1, 1))]):
        x, w = _ints(c.x_shape, 30 + t), _ints(c.w_shape, 40 + t)
        want = _scipy_ref(x, w, c)
        y, _ = fwd(x, w, c)
        _check(y.shape == want.shape and np.array_equal(y, want), "N-D case %d differs" % t)


def pin_torch_float64(fwd, bwd):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(5)
    for c, op in [(NdShape(2, 3, 2, (19,), (4,), (2,), (2,), (3,)), F.conv1d),
                  (NdShape(1, 2, 3, (7, 6, 8), (3, 2, 3), (1, 1, 0), (1, 2, 1), (2, 1, 1)), F.conv3d)]:
        x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
        w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
        dy = rng.uniform(-1, 1, c.y_shape).astype(np.float32)
        wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
        yt = op(torch.from_numpy(x.astype(np.float64)), wt, stride=c.stride, padding=c.pad,
                dilation=c.dilation)
        yt.backward(torch.from_numpy(dy.astype(np.float64)))
        y, S = fwd(x, w, c)
        _check(y.shape == tuple(yt.shape), "shape differs from torch")
        _check(np.all(np.abs(y - yt.detach().numpy()) <= 2 * c.crs * 2.0 ** -53 * S + 1e-300),
               "forward differs from torch")
        g, Sg = bwd(x, dy, c)
        terms = c.batch * c.vol_out
        _check(np.all(np.abs(g - wt.grad.numpy()) <= 2 * terms * 2.0 ** -53 * Sg + 1e-300),
               "filter gradient differs from torch")


def pin_adjoint(fwd, bwd):
    """<conv(x, w), dy> = <w, dW(x, dy)> for several w (exact on integers)."""
    rng = np.random.default_rng(7)
    for c in [NdShape(2, 2, 2, (5, 6, 4), (2, 3, 2), (1, 1, 0), (1, 2, 1), (1, 1, 2)),
              NdShape(1, 2, 2, (4, 3, 5, 4), (2, 2, 3, 2), (0, 1, 1, 0), (1, 1, 2, 1), (2, 1, 1, 1))]:
        x, dy = _ints(c.x_shape, 50), _ints(c.y_shape, 51)
        dW, _ = bwd(x, dy, c)
        for _ in range(3):
            w = rng.integers(-3, 4, c.w_shape).astype(np.float32)
            y, _ = fwd(x, w, c)
            lhs = float(np.sum(y * dy.astype(np.float64)))
            rhs = float(np.sum(w.astype(np.float64) * dW))
            _check(lhs == rhs, "adjoint identity fails (%s)" % (c.size,))


def pin_all_ones_4d(fwd, bwd):
    c = NdShape(1, 2, 1, (4, 5, 3, 6), (2, 3, 2, 3), (1, 1, 1, 2), (1, 2, 1, 2), (2, 1, 1, 1))
    y, S = fwd(np.ones(c.x_shape, np.float32), np.ones(c.w_shape, np.float32), c)

    def count(o, d):
        return sum(1 for k in range(c.kernel[d])
                   if 0 <= o * c.stride[d] - c.pad[d] + k * c.dilation[d] < c.size[d])

    for o in np.ndindex(*c.out):
        want = c.cin * np.prod([count(o[d], d) for d in range(4)])
        _check(y[(0, 0) + o] == want and S[(0, 0) + o] == want, "all-ones at %s" % (o,))


ALL_PINS = [pin_two_dims_is_the_2d_oracle, pin_one_dim_numpy, pin_three_four_dims_scipy,
            pin_torch_float64, pin_adjoint, pin_all_ones_4d]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_real_fwd, _real_bwd)


# ---------------------------------------------------------------- mutants --

def _mutant(name):
    def spatial_axes_reversed(x, w, c):     # filter taps indexed in the wrong dimension order
        if len(set(c.kernel)) != 1:
            return _real_fwd(x, w, c)
        axes = (0, 1) + tuple(range(c.nd + 1, 1, -1))
        return _real_fwd(x, np.ascontiguousarray(w.transpose(axes)), c)

    def last_dilation_ignored(x, w, c):
        if c.dilation[-1] == 1:
            return _real_fwd(x, w, c)
        c2 = NdShape(c.batch, c.cin, c.cout, c.size, c.kernel, c.pad, c.stride,
                     c.dilation[:-1] + (1,))
        y, S = _real_fwd(x, w, c2)
        sl = (slice(None), slice(None)) + tuple(slice(0, o) for o in c.out)
        return np.ascontiguousarray(y[sl]), np.ascontiguousarray(S[sl])

    def first_stride_ignored(x, w, c):
        if c.stride[0] == 1:
            return _real_fwd(x, w, c)
        c2 = NdShape(c.batch, c.cin, c.cout, c.size, c.kernel, c.pad, (1,) + c.stride[1:],
                     c.dilation)
        y, S = _real_fwd(x, w, c2)
        sl = (slice(None), slice(None)) + tuple(slice(0, o) for o in c.out)
        return np.ascontiguousarray(y[sl]), np.ascontiguousarray(S[sl])

    def filter_flipped(x, w, c):
        flip = (slice(None), slice(None)) + (slice(None, None, -1),) * c.nd
        return _real_fwd(x, np.ascontiguousarray(w[flip]), c)

    def grad_last_axis_flipped(x, dy, c):
        flip = (slice(None),) * (1 + c.nd) + (slice(None, None, -1),)
        return _real_bwd(x, np.ascontiguousarray(dy[flip]), c)

    fwd_m = {f.__name__: f for f in [spatial_axes_reversed, last_dilation_ignored,
                                     first_stride_ignored, filter_flipped]}
    if name in fwd_m:
        return fwd_m[name], _real_bwd
    return _real_fwd, grad_last_axis_flipped


MUTANTS = ["spatial_axes_reversed", "last_dilation_ignored", "first_stride_ignored",
           "filter_flipped", "grad_last_axis_flipped"]


@pytest.mark.parametrize("name", MUTANTS)
def test_pins_catch_planted_mistake(name):
    fwd, bwd = _mutant(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(fwd, bwd)
        except Exception:  # a wrong value, a wrong shape or a crash all count as caught
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name


# ------------------------------------------------------- other properties --

def test_matrix_route_equals_direct_bitwise():
    rng = np.random.default_rng(3)
    for c in [NdShape(2, 2, 3, (5, 6, 4), (2, 3, 2), (1, 1, 0), (1, 2, 1), (1, 1, 2)),
              NdShape(1, 2, 2, (4, 3, 5, 4), (2, 2, 3, 2), (0, 1, 1, 0), (1, 1, 2, 1), (2, 1, 1, 1)),
              NdShape(1, 3, 2, (11,), (3,), (1,), (2,), (2,))]:
        x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
        w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
        y, _ = ond.fwd(x, w, c)
        for n in range(c.batch):
            C, _ = oracle.gemm_f32(np.ascontiguousarray(w.reshape(c.cout, c.crs)), ond.im2col(x, c, n))
            assert np.array_equal(C, y[n].reshape(c.cout, c.vol_out))


def test_two_dim_matrix_equals_2d_matrix():
    rng = np.random.default_rng(4)
    c = NdShape(2, 3, 1, (9, 7), (3, 4), (1, 2), (2, 1), (1, 2))
    c2 = oc.ConvShape(2, 3, 9, 7, 1, 3, 4, 1, 2, 2, 1, 1, 2)
    x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
    assert np.array_equal(ond.im2col(x, c, 1), oc.im2col(x, c2, 1))


def test_invalid_shapes():
    x = np.zeros((1, 1, 4, 4, 4), np.float32)
    w = np.zeros((1, 1, 3, 3, 3), np.float32)
    with pytest.raises(ValueError):
        ond.fwd(x, w, NdShape(1, 1, 1, (4, 4, 4), (3, 3, 3), (0, 0, 0), (1, 0, 1)))
    with pytest.raises(ValueError):
        ond.fwd(x, w, NdShape(1, 1, 1, (4, 4, 4), (3, 3, 3), (0, 0, 0), (1, 1, 1), (1, 2, 1)))
    with pytest.raises(ValueError):
        NdShape(1, 1, 1, (4, 4), (3,))
