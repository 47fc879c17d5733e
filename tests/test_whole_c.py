"""Whole-output parity at every full-size workload, in the launch configuration
the benchmark times (the default dispatch), and element-wise checks of the
paths only large grids and long K loops reach.

The pass criterion of the product is the maximum over ALL entries (i, j) of
|C - C_ref| / S with S = sum_k |A_ik| |B_kj| ("Learning to develop for GPUs
through the GEMM operation", section "Matrix product", defines C_ref): a fault
confined to one block of C must not slip through, so these tests run the
threaded oracle over the whole product instead of sampled positions.

  * random operands of the workload (its own seeded distribution): the ratio
    over all M*N entries within 1e-5 (fp32) or 4e-3 (bf16 inputs), and a
    diagnostic printed when it exceeds 1e-6;
  * integer-valued operands of the same shape: every partial sum is an exact
    integer, so the whole C equals the oracle bit for bit whatever the
    summation order.
"""
from __future__ import annotations

import time

import numpy as np
import pytest

import dense_gemm_03_amd as dg
import oracle
from dense_gemm_03_amd import workloads as wl
from tests.gpu_util import DIAGNOSTIC, TOL, log, report, run, to_device

pytestmark = pytest.mark.gpu

F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16


def _ints(shape, seed, bf16):
    return wl.small_int_bf16_bits(shape, seed) if bf16 else wl.small_int_f32(shape, seed)


def _oracle(A, B, with_s=True):
    fn = oracle.gemm_f32 if A.dtype == np.float32 else oracle.gemm_bf16
    t = time.perf_counter()
    out = fn(A, B, with_s=with_s)
    log("  oracle %dx%dx%d on %d threads: %.1f s" % (
        A.shape[0], B.shape[1], A.shape[1], oracle.default_threads(), time.perf_counter() - t))
    return out


def _exact_whole(C, A, B, what):
    C_ref = _oracle(A, B, with_s=False)
    bad = np.flatnonzero(C.astype(np.float64) != C_ref)
    if bad.size:
        i, j = divmod(int(bad[0]), C.shape[1])
        raise AssertionError("%s: %d of %d entries differ, first (%d,%d): gpu %r oracle %r" % (
            what, bad.size, C.size, i, j, C[i, j], C_ref[i, j]))
    report("whole C, integer operands, %s: all %d x %d = %d entries equal the oracle bit for bit"
           % (what, C.shape[0], C.shape[1], C.size))


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_whole_c_random_within_tolerance(name):
    w = wl.WORKLOADS[name]
    log("[%s] drawing %dx%dx%d operands (%s)" % (name, w.M, w.N, w.K, w.dist))
    A, B = w.operands()
    cfg_id = dg.gemm_select_config(F32 if w.dtype == "f32" else BF16, w.M, w.N, w.K)
    log("[%s] GPU, default dispatch (%s)" % (
        name, dg.gemm_config_name(F32 if w.dtype == "f32" else BF16, cfg_id)))
    C = run(A, B).cpu().numpy()
    C_ref, S = _oracle(A, B)
    del A, B
    ratio, zeros_ok = oracle.max_error_ratio(C, C_ref, S)
    report("whole C, random operands, %s: max over all %d x %d = %d entries of |C-C_ref|/S = "
           "%.3e (tol %.0e)%s" % (name, w.M, w.N, C.size, ratio, TOL[w.dtype],
                                  "  [diagnostic: above %.0e]" % DIAGNOSTIC
                                  if ratio > DIAGNOSTIC else ""))
    assert zeros_ok
    assert ratio <= TOL[w.dtype]


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_whole_c_exact_integers(name):
    w = wl.WORKLOADS[name]
    bf16 = w.dtype == "bf16"
    log("[%s] integer operands %dx%dx%d" % (name, w.M, w.N, w.K))
    A, B = _ints((w.M, w.K), w.seed + 7, bf16), _ints((w.K, w.N), w.seed + 8, bf16)
    C = run(A, B).cpu().numpy()
    _exact_whole(C, A, B, name)


def _config(dtype, name):
    for c in range(dg.gemm_num_configs(dtype)):
        if dg.gemm_config_name(dtype, c) == name:
            return c
    raise KeyError(name)


@pytest.mark.parametrize("name,bk", [("bf16_256x256x32_w4x2_s4", 32), ("bf16_256x256x64_w4x2_s2", 64)])
def test_rotated_k_order_interior_blocks_exact(name, bk):
    """The 32-deep bf16 256x256 blocks walk their k-tiles from a start tile
    that depends on the block's position once a block holds at least 32
    interior k-tiles (the 64-deep blocks walk the same long loops in order).
    512 x 512 x 64 BK (64 k-tiles) puts four interior blocks, with different
    start tiles, on that path, and 768 x 1024 x 33 BK exactly 33; integer
    operands make the whole C exact."""
    cfg = _config(BF16, name)
    for (M, N, K, seed) in [(512, 512, 64 * bk, 1), (768, 1024, 33 * bk, 2)]:
        A, B = _ints((M, K), 40 + seed, True), _ints((K, N), 50 + seed, True)
        log("%s %dx%dx%d (%d k-tiles per block)" % (name, M, N, K, K // bk))
        C = run(A, B, cfg=cfg).cpu().numpy()
        _exact_whole(C, A, B, "%s rotated %dx%dx%d" % (name, M, N, K))
    # random values within the tolerance on the same path
    K = 64 * bk
    A, B = wl.normal_bf16_bits((1024, K), 3), wl.normal_bf16_bits((K, 1024), 4)
    C = run(A, B, cfg=cfg).cpu().numpy()
    C_ref, S = _oracle(A, B)
    ratio, zeros_ok = oracle.max_error_ratio(C, C_ref, S)
    report("whole C, random operands, %s rotated k-order 1024x1024x%d: max over all entries of "
           "|C-C_ref|/S = %.3e" % (name, K, ratio))
    assert zeros_ok and ratio <= TOL["bf16"]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_many_blocks_xcd_renumbering_exact(bf16):
    """Grids of at least 1024 blocks, a multiple of 8, so the XCD-aware
    renumbering of block ids runs over many rounds of the chip; every block
    of C is compared element by element (integer operands: exact)."""
    dtype = BF16 if bf16 else F32
    name = "bf16_64x64x64_w2x2_s2" if bf16 else "f32_64x64_w2x2_s2"
    cfg = _config(dtype, name)
    for (M, N, K) in [(2048, 2048, 512), (1024, 4096 + 64, 320)]:
        blocks = -(-M // 64) * -(-N // 64)
        log("%s %dx%dx%d: %d blocks" % (name, M, N, K, blocks))
        assert blocks >= 1024 and blocks % 8 == 0
        A, B = _ints((M, K), 60 + M % 7, bf16), _ints((K, N), 70 + N % 7, bf16)
        C = run(A, B, cfg=cfg).cpu().numpy()
        _exact_whole(C, A, B, "%s %dx%dx%d" % (name, M, N, K))


@pytest.mark.parametrize("case", [
    ("f32", False, False, 4097, 4095, 256, 1.0, 0.0),
    ("f32", True, True, 4099, 4098, 200, 2.0, -1.0),
    ("f32", False, True, 4095, 4100, 160, 1.0, 1.0),
    ("bf16", False, False, 4097, 4095, 192, 1.0, 0.0),
    ("bf16", True, False, 4100, 4099, 128, -1.0, 2.0),
    ("bf16", False, False, 3080, 3075, 192, 1.0, 0.0),
    ("bf16", False, True, 3075, 3090, 160, 2.0, -1.0),
], ids=lambda c: "%s-%s%s-%dx%dx%d" % (c[0], "T" if c[1] else "N", "T" if c[2] else "N",
                                        c[3], c[4], c[5]))
def test_thin_remainders_run_apart_exact(case):
    """Large products whose last block row or column would hold only a few
    rows (columns): the dispatcher runs the full 256 x 256 (or 192 x 256)
    blocks as one product and the thin strips as products of their own.  Every entry of C,
    for transposed operands and alpha/beta too, equals the oracle's exact
    value (integer operands and C)."""
    import torch
    dt, ta, tb, M, N, K, alpha, beta = case
    bf16 = dt == "bf16"
    dtype = BF16 if bf16 else F32
    cfg = dg.gemm_select_config_ex(dtype, int(ta), int(tb), M, N, K)
    assert dg.gemm_config_name(dtype, cfg).endswith(("256x256_w4x2_s2", "256x256x32_w4x2_s4",
                                                     "256x256x64_w4x2_s2", "192x256x64_w2x4_s2"))
    A = _ints((K, M) if ta else (M, K), 80 + M % 5, bf16)
    B = _ints((N, K) if tb else (K, N), 90 + N % 5, bf16)
    C0 = np.random.default_rng(K).integers(-9, 10, size=(M, N)).astype(np.float32)
    Ad, Bd = to_device(A), to_device(B)
    C = torch.from_numpy(C0).to("cuda:0")
    dg.gemm(Ad, Bd, out=C, alpha=alpha, beta=beta, transa=ta, transb=tb)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    want, _ = oracle.gemm_general(A, B, alpha, beta, C0.astype(np.float64) if beta else None, ta,
                                  tb, kind=dt)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "%d of %d entries differ, first at %s" % (
        bad.size, got.size, divmod(int(bad[0]), N))
    report("whole C, integer operands, thin remainders %s %s%s %dx%dx%d alpha %g beta %g: all %d "
           "entries equal the oracle bit for bit" % (dt, "T" if ta else "N", "T" if tb else "N",
                                                      M, N, K, alpha, beta, got.size))
