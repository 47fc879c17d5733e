"""The convolution oracle against its pins (CPU only).

``oracle.conv`` is direct 2-D convolution (cross-correlation form, channel-
first, stride / zero padding / dilation) and its filter gradient, from "Three
X's: a new level of working with large convolutions in PyTorch for model
training".  Pins that do not retype the definition:
  * the page's worked index example (tests/golden/conv_worked_example.txt);
  * single-channel cases that reduce to scipy's 2-D cross-correlation, exact
    on integers, with stride as subsampling and dilation as a zero-stuffed
    filter;
  * agreement with torch's float64 conv2d within the fp64 summation bound;
  * 1x1 filters reduce to the pinned GEMM oracle, bit for bit;
  * all-ones closed form (the count of in-image taps);
  * the filter gradient is the adjoint of the forward map in the filter:
    <conv(x, w), dy> = <w, dW(x, dy)>, exact on integers, plus its scipy form;
  * the im2col matrix times the filters equals the direct convolution, bit for bit.
Mutants with planted mistakes each fail at least one pin.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle import conv as oc
from oracle.conv import ConvShape

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "conv_worked_example.txt")


class PinFailure(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise PinFailure(msg)


def _ints(shape, seed, lo=-3, hi=3):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def _real_fwd(x, w, c):
    return oc.conv2d_fwd(x, w, c, threads=3)


def _real_bwd(x, dy, c):
    return oc.conv2d_bwd_weight(x, dy, c, threads=3)


# ------------------------------------------------------------------- pins --

def read_worked_example():
    page, reading = {}, {"o": {}, "o7tap": []}
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "page":
            page[f[1]] = [int(v) for v in f[2:]]
        elif f[1] == "o":
            reading["o"][int(f[2])] = (int(f[3]), int(f[4]))
        elif f[1] == "o7tap":
            reading["o7tap"].append(tuple(int(v) for v in f[2:]))
        else:
            reading[f[1]] = [int(v) for v in f[2:]]
    return page, reading


def pin_worked_example(fwd, bwd):
    """The page's example: 3x3 image, 3x3 filter, nine results, o7 at [2, 0].
    With image values 2^(3i+j) and a one-hot filter at tap (r, s), the result
    at [p, q] is the single image value that tap reads, so every output names
    the image position it used; the fixture's window of o7 must come out."""
    page, rd = read_worked_example()
    c = ConvShape(1, 1, *page["image"], 1, *page["filter"], ph=rd["pad"][0], pw=rd["pad"][1],
                  sh=rd["stride"][0], sw=rd["stride"][1])
    _check(c.p * c.q == page["results"][0], "nine results expected")
    x = (2.0 ** np.arange(9)).reshape(1, 1, 3, 3).astype(np.float32)
    # identifiers o1..o9 -> coordinates, and o7 -> [2, 0] as the page states
    for k, (p, q) in rd["o"].items():
        _check(divmod(k - 1, c.q) == (p, q), "o%d maps to %s" % (k, (p, q)))
    p7, q7 = rd["o"][7]
    _check([p7, q7] == page["o7"], "o7 must be [2, 0]")
    for (r, s, iy, ix, inside) in rd["o7tap"]:
        w = np.zeros((1, 1, 3, 3), dtype=np.float32)
        w[0, 0, r, s] = 1.0
        y, _ = fwd(x, w, c)
        want = 2.0 ** (3 * iy + ix) if inside else 0.0
        _check(y[0, 0, p7, q7] == want, "tap (%d,%d) of o7 reads [%d,%d]" % (r, s, iy, ix))


def pin_scipy_single_channel(fwd, bwd):
    """One channel in and out: the oracle equals scipy's 2-D cross-correlation
    of the zero-padded image (exact on integers); stride subsamples the unit-
    stride result; dilation is the same correlation with a zero-stuffed filter."""
    for t, (H, W, R, S, ph, pw, sh, sw, dh, dw) in enumerate(
            [(7, 9, 3, 2, 0, 0, 1, 1, 1, 1), (8, 6, 3, 3, 1, 2, 1, 1, 1, 1),
             (11, 10, 3, 4, 2, 1, 2, 3, 1, 1), (12, 13, 3, 2, 1, 0, 1, 2, 2, 3),
             (5, 5, 5, 5, 4, 4, 1, 1, 1, 1)]):
        x = _ints((1, 1, H, W), 40 + t)
        w = _ints((1, 1, R, S), 50 + t)
        c = ConvShape(1, 1, H, W, 1, R, S, ph, pw, sh, sw, dh, dw)
        wd = np.zeros(((R - 1) * dh + 1, (S - 1) * dw + 1))
        wd[::dh, ::dw] = w[0, 0]
        xp = np.pad(x[0, 0].astype(np.float64), ((ph, ph), (pw, pw)))
        full = scipy.signal.correlate2d(xp, wd, mode="valid")
        want = full[::sh, ::sw]
        y, _ = fwd(x, w, c)
        _check(y.shape[2:] == want.shape, "output size %s vs %s" % (y.shape[2:], want.shape))
        _check(np.array_equal(y[0, 0], want), "single-channel case %d differs from scipy" % t)


def pin_multi_channel_sum(fwd, bwd):
    """C_in > 1: the sum over input channels of single-channel correlations;
    each output channel uses its own filter bank (exact on integers)."""
    for t, c in enumerate([ConvShape(2, 3, 6, 7, 4, 3, 2, 1, 1), ConvShape(1, 3, 5, 5, 3, 3, 3, 1, 1)]):
        x, w = _ints(c.x_shape, 61 + t), _ints(c.w_shape, 62 + t)
        y, _ = fwd(x, w, c)
        for n in range(c.batch):
            for co in range(c.cout):
                want = sum(scipy.signal.correlate2d(
                    np.pad(x[n, ci].astype(np.float64), 1), w[co, ci].astype(np.float64),
                    mode="valid") for ci in range(c.cin))
                _check(np.array_equal(y[n, co], want), "channel sum (n=%d co=%d)" % (n, co))


def pin_one_by_one_is_gemm(fwd, bwd):
    """1x1 filters, no padding, unit stride: y[n] = W . X[n] as matrices, and
    the oracle sums in the same ascending channel order as the GEMM oracle,
    so the results agree bit for bit on random reals."""
    rng = np.random.default_rng(7)
    c = ConvShape(2, 5, 4, 6, 3, 1, 1)
    x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
    w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
    y, S = fwd(x, w, c)
    for n in range(c.batch):
        C, Sg = oracle.gemm_f32(np.ascontiguousarray(w.reshape(3, 5)),
                                np.ascontiguousarray(x[n].reshape(5, 24)))
        _check(np.array_equal(y[n].reshape(3, 24), C) and np.array_equal(S[n].reshape(3, 24), Sg),
               "1x1 convolution differs from the GEMM")


def pin_all_ones(fwd, bwd):
    """x = 1, w = 1: each output counts the filter taps that land inside the
    image, C_in times; that count is the product of the per-axis counts."""
    c = ConvShape(1, 2, 5, 7, 1, 3, 4, 2, 1, 2, 1, 1, 2)

    def count(p, size, pad, k, st, dil):
        return sum(1 for t in range(k) if 0 <= p * st - pad + t * dil < size)

    y, S = fwd(np.ones(c.x_shape, np.float32), np.ones(c.w_shape, np.float32), c)
    for p in range(c.p):
        for q in range(c.q):
            want = c.cin * count(p, c.h, c.ph, c.r, c.sh, c.dh) * count(q, c.w, c.pw, c.s, c.sw, c.dw)
            _check(y[0, 0, p, q] == want and S[0, 0, p, q] == want, "all-ones at %s" % ((p, q),))


def pin_torch_float64(fwd, bwd):
    """Random reals against torch's float64 conv2d (and its filter gradient by
    autograd), within twice the fp64 summation bound."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    for c in [ConvShape(2, 3, 9, 8, 4, 3, 3, 1, 1), ConvShape(1, 2, 11, 10, 3, 4, 3, 2, 1, 2, 3, 1, 2)]:
        x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
        w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
        dy = rng.uniform(-1, 1, c.y_shape).astype(np.float32)
        xt = torch.from_numpy(x.astype(np.float64))
        wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
        yt = torch.nn.functional.conv2d(xt, wt, stride=(c.sh, c.sw), padding=(c.ph, c.pw),
                                        dilation=(c.dh, c.dw))
        yt.backward(torch.from_numpy(dy.astype(np.float64)))
        y, S = fwd(x, w, c)
        _check(y.shape == tuple(yt.shape), "output shape differs from torch")
        _check(np.all(np.abs(y - yt.detach().numpy()) <= 2 * c.crs * 2.0 ** -53 * S + 1e-300),
               "forward differs from torch")
        dw, Sw = bwd(x, dy, c)
        terms = c.batch * c.p * c.q
        _check(np.all(np.abs(dw - wt.grad.numpy()) <= 2 * terms * 2.0 ** -53 * Sw + 1e-300),
               "filter gradient differs from torch")


def pin_bwd_adjoint(fwd, bwd):
    """<conv(x, w), dy> = <w, dW(x, dy)> for every w: the filter gradient is
    the adjoint of the forward map in w.  Small integers keep every sum exact,
    and a few random w (plus one-hot w) make the identity a full check."""
    c = ConvShape(2, 3, 7, 6, 2, 3, 2, 1, 2, 2, 1, 1, 2)
    x, dy = _ints(c.x_shape, 81), _ints(c.y_shape, 82)
    dW, _ = bwd(x, dy, c)
    rng = np.random.default_rng(83)
    ws = [rng.integers(-3, 4, c.w_shape).astype(np.float32) for _ in range(3)]
    for idx in [(0, 0, 0, 0), (1, 2, 2, 1), (0, 1, 1, 0)]:
        e = np.zeros(c.w_shape, np.float32)
        e[idx] = 1.0
        ws.append(e)
    for w in ws:
        y, _ = fwd(x, w, c)
        lhs = float(np.sum(y * dy.astype(np.float64)))
        rhs = float(np.sum(w.astype(np.float64) * dW))
        _check(lhs == rhs, "adjoint identity fails: %r vs %r" % (lhs, rhs))


def pin_bwd_scipy(fwd, bwd):
    """Unit stride and dilation: dW[co][ci] is the cross-correlation of the
    padded image channel with the output-gradient channel, summed over images."""
    c = ConvShape(2, 2, 6, 5, 3, 3, 2, 1, 1)
    x, dy = _ints(c.x_shape, 91), _ints(c.y_shape, 92)
    dW, _ = bwd(x, dy, c)
    for co in range(c.cout):
        for ci in range(c.cin):
            want = sum(scipy.signal.correlate2d(
                np.pad(x[n, ci].astype(np.float64), ((c.ph, c.ph), (c.pw, c.pw))),
                dy[n, co].astype(np.float64), mode="valid") for n in range(c.batch))
            _check(np.array_equal(dW[co, ci], want), "filter gradient (%d,%d)" % (co, ci))


ALL_PINS = [pin_worked_example, pin_scipy_single_channel, pin_multi_channel_sum,
            pin_one_by_one_is_gemm, pin_all_ones, pin_torch_float64, pin_bwd_adjoint,
            pin_bwd_scipy]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_real_fwd, _real_bwd)


# ---------------------------------------------------------------- mutants --

def _mutant(name):
    def flipped_filter(x, w, c):       # true convolution instead of cross-correlation
        return _real_fwd(x, np.ascontiguousarray(w[:, :, ::-1, ::-1]), c)

    def taps_transposed(x, w, c):      # r and s exchanged
        if c.r != c.s:
            return _real_fwd(x, w, c)
        return _real_fwd(x, np.ascontiguousarray(w.transpose(0, 1, 3, 2)), c)

    def dilation_ignored(x, w, c):     # taps one pixel apart whatever the dilation
        if (c.dh, c.dw) == (1, 1):
            return _real_fwd(x, w, c)
        c2 = ConvShape(c.batch, c.cin, c.h, c.w, c.cout, c.r, c.s, c.ph, c.pw, c.sh, c.sw, 1, 1)
        y, S = _real_fwd(x, w, c2)
        return np.ascontiguousarray(y[:, :, :c.p, :c.q]), np.ascontiguousarray(S[:, :, :c.p, :c.q])

    def padding_shift_lost(x, w, c):   # pads only one side: the window starts at p*sh
        if c.ph == 0 and c.pw == 0:
            return _real_fwd(x, w, c)
        xp = np.zeros((c.batch, c.cin, c.h + c.ph, c.w + c.pw), dtype=x.dtype)
        xp[:, :, :c.h, :c.w] = x
        c2 = ConvShape(c.batch, c.cin, c.h + c.ph, c.w + c.pw, c.cout, c.r, c.s, 0, 0,
                       c.sh, c.sw, c.dh, c.dw)
        y, S = _real_fwd(xp, w, c2)
        return y[:, :, :c.p, :c.q], S[:, :, :c.p, :c.q]

    def channel_order_swapped(x, w, c):   # filters indexed [ci][co]
        if c.cin != c.cout:
            return _real_fwd(x, w, c)
        return _real_fwd(x, np.ascontiguousarray(w.transpose(1, 0, 2, 3)), c)

    def grad_dy_flipped(x, dy, c):
        return _real_bwd(x, np.ascontiguousarray(dy[:, :, ::-1, ::-1]), c)

    def grad_images_dropped(x, dy, c):    # only the first image accumulated
        if c.batch < 2:
            return _real_bwd(x, dy, c)
        c1 = ConvShape(1, *[getattr(c, f) for f in ("cin", "h", "w", "cout", "r", "s", "ph", "pw",
                                                      "sh", "sw", "dh", "dw")])
        return _real_bwd(np.ascontiguousarray(x[:1]), np.ascontiguousarray(dy[:1]), c1)

    fwd_mutants = {f.__name__: f for f in [flipped_filter, taps_transposed,
                                           dilation_ignored, padding_shift_lost,
                                           channel_order_swapped]}
    bwd_mutants = {f.__name__: f for f in [grad_dy_flipped, grad_images_dropped]}
    if name in fwd_mutants:
        return fwd_mutants[name], _real_bwd
    return _real_fwd, bwd_mutants[name]


MUTANTS = ["flipped_filter", "taps_transposed", "dilation_ignored", "padding_shift_lost",
           "channel_order_swapped", "grad_dy_flipped", "grad_images_dropped"]


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

def test_im2col_route_equals_direct_convolution_bitwise():
    """W (C_out x C_in R S) times the convolution matrix (C_in R S x P Q) is the
    direct convolution: same terms, same ascending (ci, r, s) order, and the
    padding contributes exact zeros, so the two agree bit for bit."""
    rng = np.random.default_rng(5)
    for c in [ConvShape(2, 3, 9, 8, 4, 3, 3, 1, 1), ConvShape(1, 2, 12, 11, 3, 4, 3, 2, 1, 2, 3, 1, 2),
              ConvShape(1, 1, 3, 3, 1, 3, 3, 1, 1)]:
        x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
        w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
        y, _ = oc.conv2d_fwd(x, w, c)
        for n in range(c.batch):
            cols = oc.im2col(x, c, n)
            C, _ = oracle.gemm_f32(np.ascontiguousarray(w.reshape(c.cout, c.crs)), cols)
            assert np.array_equal(C, y[n].reshape(c.cout, c.p * c.q))


def test_im2col_worked_example_column():
    """Column o7 of the page's example holds the four in-image values of its
    window and zeros for the padding, in tap order."""
    page, rd = read_worked_example()
    c = ConvShape(1, 1, 3, 3, 1, 3, 3, 1, 1)
    x = (np.arange(9, dtype=np.float32) + 1).reshape(1, 1, 3, 3)
    col = oc.im2col(x, c)[:, 6]
    want = [x[0, 0, iy, ix] if inside else 0.0 for (r, s, iy, ix, inside) in rd["o7tap"]]
    assert list(col) == want


def test_im2col_leading_dimension_and_bf16_bits():
    rng = np.random.default_rng(9)
    c = ConvShape(2, 2, 5, 6, 1, 2, 3, 1, 0, 1, 2)
    x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
    tight = oc.im2col(x, c, 1)
    padded = oc.im2col(x, c, 1, ld=tight.shape[1] + 5)
    assert np.array_equal(padded[:, :tight.shape[1]], tight) and np.all(padded[:, tight.shape[1]:] == 0)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oc.im2col(bits, c, 1), (tight.view(np.uint32) >> 16).astype(np.uint16))


def test_bf16_kind_matches_f32_kind():
    c = ConvShape(2, 2, 6, 7, 3, 3, 2, 1, 1, 2, 1)
    x, w, dy = _ints(c.x_shape, 1) / 4, _ints(c.w_shape, 2) / 8, _ints(c.y_shape, 3) / 2
    bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    yf = oc.conv2d_fwd(x.astype(np.float32), w.astype(np.float32), c)
    yb = oc.conv2d_fwd(bits(x), bits(w), c)
    assert np.array_equal(yf[0], yb[0]) and np.array_equal(yf[1], yb[1])
    gf = oc.conv2d_bwd_weight(x.astype(np.float32), dy.astype(np.float32), c)
    gb = oc.conv2d_bwd_weight(bits(x), bits(dy), c)
    assert np.array_equal(gf[0], gb[0]) and np.array_equal(gf[1], gb[1])


def test_entries_match_full_bitwise():
    rng = np.random.default_rng(11)
    c = ConvShape(3, 2, 9, 7, 4, 3, 2, 1, 0, 2, 1, 1, 2)
    x = rng.uniform(-1, 1, c.x_shape).astype(np.float32)
    w = rng.uniform(-1, 1, c.w_shape).astype(np.float32)
    dy = rng.uniform(-1, 1, c.y_shape).astype(np.float32)
    y, S = oc.conv2d_fwd(x, w, c)
    idx = [rng.integers(0, d, 40) for d in c.y_shape]
    ye, Se = oc.conv2d_fwd_entries(x, w, c, *idx)
    assert np.array_equal(ye, y[tuple(idx)]) and np.array_equal(Se, S[tuple(idx)])
    dw, Sw = oc.conv2d_bwd_weight(x, dy, c)
    idx = [rng.integers(0, d, 40) for d in c.w_shape]
    de, Sde = oc.conv2d_bwd_weight_entries(x, dy, c, *idx)
    assert np.array_equal(de, dw[tuple(idx)]) and np.array_equal(Sde, Sw[tuple(idx)])


def test_output_size_and_invalid_arguments():
    # the formula on hand cases, including a filter that does not fit
    assert oc.out_dim(128, 15, 31, 1, 1) == 128
    assert oc.out_dim(3, 1, 3, 1, 1) == 3
    assert oc.out_dim(10, 0, 3, 2, 1) == 4
    assert oc.out_dim(10, 1, 3, 3, 2) == 3
    assert oc.out_dim(4, 0, 3, 1, 2) == 0
    torch = pytest.importorskip("torch")
    for (H, ph, R, sh, dh) in [(7, 0, 3, 1, 1), (9, 2, 4, 3, 2), (16, 3, 5, 2, 3), (5, 4, 5, 4, 1)]:
        t = torch.nn.functional.conv2d(torch.zeros(1, 1, H, H), torch.zeros(1, 1, R, R),
                                       stride=sh, padding=ph, dilation=dh)
        assert t.shape[-1] == oc.out_dim(H, ph, R, sh, dh)
    x, w = np.zeros((1, 1, 4, 4), np.float32), np.zeros((1, 1, 3, 3), np.float32)
    for bad in [ConvShape(1, 1, 4, 4, 1, 3, 3, 0, 0, 0, 1), ConvShape(1, 1, 4, 4, 1, 3, 3, -1, 0),
                ConvShape(1, 1, 4, 4, 1, 3, 3, 0, 0, 1, 1, 3, 1)]:
        with pytest.raises(ValueError):
            oc.conv2d_fwd(x, w, bad)
