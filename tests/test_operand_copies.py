"""Loads that run past M or N, and bf16 operands whose rows are not 4-byte
aligned, on integer operands bit for bit against the oracle
("Learning to develop for GPUs through the GEMM operation", sections "Matrix
product" and "Generalized matrix multiplication GEMM", define the results):

  * operands whose rows are 16-byte aligned, with an odd M (A^T) or N (B)
    along the rows: the loads run on to the next 16 bytes, into the row's
    padding, which holds NaN here and must never reach a stored output;
  * bf16 operands at odd pitches or 2-byte-aligned addresses, in products
    large enough that the dispatcher first copies them into 16-byte-aligned
    rows (gemm_operand_copy_bytes > 0);
  * the same under graph capture: a stream without the copy buffer runs the
    captured product on the operands in place, a warmed stream copies inside
    the graph; every replay equals the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_03_amd as dg
import oracle
from dense_gemm_03_amd import workloads as wl
from tests.gpu_util import log, report
from tests.test_variants import BF16_NAN, TNAME, TRANS, check_exact_ex, run_ex

pytestmark = pytest.mark.gpu

F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16


def _ints(shape, seed, bf16):
    return wl.small_int_bf16_bits(shape, seed) if bf16 else wl.small_int_f32(shape, seed)


def _device(x, ld, offset=0):
    """x (numpy; uint16 = bf16 bits) on cuda:0 in a NaN-filled buffer whose
    rows hold `ld` elements, starting `offset` elements into each row; the
    returned view has x's shape and leading dimension ld."""
    import torch
    rows, cols = x.shape
    if x.dtype == np.uint16:
        buf = np.full((rows, ld), BF16_NAN, dtype=np.uint16)
        buf[:, offset:offset + cols] = x
        t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16)
    else:
        buf = np.full((rows, ld), np.nan, dtype=np.float32)
        buf[:, offset:offset + cols] = x
        t = torch.from_numpy(buf)
    return t.to("cuda:0")[:, offset:offset + cols]


def _run(A, B, ta, tb, lda, ldb, cfg=None, a_off=0, b_off=0):
    import torch
    Ad, Bd = _device(A, lda, a_off), _device(B, ldb, b_off)
    M = A.shape[1] if ta else A.shape[0]
    N = B.shape[0] if tb else B.shape[1]
    C = torch.full((M, N), float("nan"), device="cuda:0")
    dg.gemm(Ad, Bd, out=C, cfg=cfg, transa=ta, transb=tb)
    torch.cuda.synchronize()
    return C.cpu().numpy(), Ad, Bd


def _rup(x, m):
    return -(-x // m) * m


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_aligned_rows_odd_extents_every_config(bf16):
    """Every entry and operand form it is built for, rows at a multiple of 16
    bytes (8 more elements than the row rounded up), odd M and N: the blocks
    at the M and N edges load whole 16-byte chunks of the padding, NaN here,
    which feed only outputs that are never stored."""
    dtype = BF16 if bf16 else F32
    vec = 8 if bf16 else 4
    for cfg in range(dg.gemm_num_configs(dtype)):
        name = dg.gemm_config_name(dtype, cfg)
        mask = dg.gemm_config_layouts(dtype, cfg)
        for ta, tb in TRANS:
            if not mask & (1 << (2 * ta + tb)):
                continue
            for t, (M, N, K) in enumerate([(301, 203, 166), (517, 259, 130)]):
                A = _ints((K, M) if ta else (M, K), 70 + t, bf16)
                B = _ints((N, K) if tb else (K, N), 80 + t, bf16)
                lda, ldb = _rup(A.shape[1], vec) + 8, _rup(B.shape[1], vec) + 8
                what = "%s %s %dx%dx%d lda %d ldb %d" % (name, TNAME[ta, tb], M, N, K, lda, ldb)
                log(what)
                C, _, _ = _run(A, B, ta, tb, lda, ldb, cfg=cfg)
                check_exact_ex(C.astype(np.float64), A, B, ta, tb, 1.0, 0.0, None, False, what)


def test_copied_operands_exact_every_form():
    """bf16 products the dispatcher runs on row-aligned copies: odd pitches in
    every operand form, A at an address 2 bytes past a 4-byte boundary (even
    pitch), and alpha/beta with bf16 C."""
    M, N, K = 1537, 1539, 1541
    for ta, tb in TRANS:
        A = _ints((K, M) if ta else (M, K), 90, True)
        B = _ints((N, K) if tb else (K, N), 91, True)
        lda, ldb = A.shape[1], B.shape[1]
        C, Ad, Bd = _run(A, B, ta, tb, lda, ldb)
        copied = dg.gemm_operand_copy_bytes(BF16, int(ta), int(tb), M, N, K, Ad.data_ptr(), lda,
                                            Bd.data_ptr(), ldb)
        assert copied == (_rup(A.shape[0] * _rup(A.shape[1], 8) * 2, 256) +
                          B.shape[0] * _rup(B.shape[1], 8) * 2)
        what = "copied %s %dx%dx%d (odd pitches, %d bytes of copies)" % (
            TNAME[ta, tb], M, N, K, copied)
        log(what)
        check_exact_ex(C.astype(np.float64), A, B, ta, tb, 1.0, 0.0, None, False, what)
    # A 2 bytes past a 4-byte boundary, even pitch: A alone is copied
    A, B = _ints((M, K + 1), 92, True), _ints((K + 1, N + 1), 93, True)
    C, Ad, Bd = _run(A, B, False, False, K + 3, _rup(N + 1, 8), a_off=1)
    assert Ad.data_ptr() % 4 == 2
    copied = dg.gemm_operand_copy_bytes(BF16, 0, 0, M, N + 1, K + 1, Ad.data_ptr(), K + 3,
                                        Bd.data_ptr(), _rup(N + 1, 8))
    assert copied == _rup(M * _rup(K + 1, 8) * 2, 256)
    check_exact_ex(C.astype(np.float64), A, B, False, False, 1.0, 0.0, None, False,
                   "copied A at a 2-byte-aligned address")
    # alpha, beta and bf16 C on copied operands
    C0 = np.random.default_rng(5).integers(-9, 10, size=(M, N)).astype(np.float64)
    A, B = _ints((K, M), 94, True), _ints((K, N), 95, True)
    _, raw = run_ex(A, B, True, False, 2.0, -3.0, C0, True)
    check_exact_ex(raw, A, B, True, False, 2.0, -3.0, C0, True, "copied TN alpha 2 beta -3 bf16 C")
    report("copied bf16 operands (odd pitches, every form; 2-byte-aligned A; alpha/beta with bf16 "
           "C) at %dx%dx%d: bit for bit equal to the oracle" % (M, N, K))


def test_copies_under_graph_capture():
    """A product that copies its operands, captured on a stream that has no
    copy buffer yet, runs on the operands in place inside the graph; once a
    call has run on the stream, a capture copies inside the graph.  Each graph
    is replayed three times with new operands written eagerly in between, and
    every replay equals the oracle."""
    import torch
    M, N, K = 1153, 1151, 1155                       # about 576 flops per copied byte
    A = torch.empty((M, K), dtype=torch.bfloat16, device="cuda:0")
    B = torch.empty((K, N), dtype=torch.bfloat16, device="cuda:0")
    C = torch.empty((M, N), device="cuda:0")
    assert dg.gemm_operand_copy_bytes(BF16, 0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N) > 0
    cfg = dg.gemm_select_config(BF16, M, N, K)
    assert dg.gemm_split_k(BF16, cfg, M, N, K) == 1      # no split-K workspace either way

    def fill(seed):
        a, b = _ints((M, K), seed, True), _ints((K, N), seed + 1, True)
        A.copy_(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16))
        B.copy_(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16))
        torch.cuda.synchronize()
        return a, b

    for warm in (False, True):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        if warm:
            fill(100)
            with torch.cuda.stream(s):
                dg.gemm(A, B, out=C, stream=s.cuda_stream)     # creates the copy buffer
            torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dg.gemm(A, B, out=C, stream=s.cuda_stream)
        torch.cuda.synchronize()
        for r in range(3):
            a, b = fill(200 + 10 * r + int(warm))
            C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = C.cpu().numpy().astype(np.float64)
            bad = np.flatnonzero(got != oracle.gemm_bf16(a, b, with_s=False))
            assert bad.size == 0, "%s stream, replay %d: %d entries differ" % (
                "warmed" if warm else "fresh", r, bad.size)
            log("graph on a %s stream, replay %d: equal to the oracle" % (
                "warmed" if warm else "fresh", r))
        del g
        dg.gemm_release_buffers(s.cuda_stream)
