"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and its host logic (argument checks, shape-class dispatch, split-K
planning) behaves as documented.  No call here reaches a kernel: invalid
arguments are rejected before any HIP call, and empty outputs launch nothing.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import dense_gemm_03_amd as dg
from dense_gemm_03_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gemm.h", "conv.h")]


def header_functions():
    names = set()
    for path in HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:gemm|conv2d|convnd)_\w+)\s*\(",
                                text, re.M))
    return sorted(names)


def test_library_loads_and_exports_header_symbols():
    lib = ctypes.CDLL(dg.LIB_PATH)
    names = header_functions()
    assert len(names) == 35, names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(dg.SIGNATURES)


def test_status_strings():
    assert dg.gemm_status_string(dg.GEMM_OK) == "success"
    assert dg.gemm_status_string(dg.GEMM_ERR_INVALID_ARG) == "invalid argument"
    assert dg.gemm_status_string(dg.GEMM_ERR_HIP) == "HIP runtime error"
    assert dg.gemm_status_string(dg.GEMM_ERR_NO_DEVICE) == "no HIP device"
    assert dg.gemm_status_string(dg.GEMM_ERR_OUT_OF_MEMORY) == "out of device memory"
    assert dg.gemm_status_string(dg.GEMM_ERR_INTERNAL).startswith("internal error")
    assert "captured" in dg.gemm_status_string(dg.GEMM_ERR_CAPTURING)
    assert dg.gemm_status_string(12345) == "unknown status"


def test_release_buffers_without_a_device():
    """No GPU here: releasing a stream's buffers reports the missing device
    instead of touching one."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only check")
    assert dg.gemm_release_buffers(None) == dg.GEMM_ERR_NO_DEVICE


def test_operand_copy_rule():
    """bf16 operands whose rows are not all 4-byte aligned are copied into
    zero-padded 16-byte-aligned rows when the product does 160 flops per
    copied byte of a k-contiguous operand (A, B^T) plus 56 per copied byte of
    an outer-contiguous one (A^T, B), K >= 256 and 2^26 flops.  The query
    looks at the pointers' alignment only and never reads them, so integers
    stand in for device addresses here."""
    BF16, F32 = dg.GEMM_DTYPE_BF16, dg.GEMM_DTYPE_F32
    q = dg.gemm_operand_copy_bytes
    base = 1 << 20
    rup = lambda x, m: -(-x // m) * m
    # odd pitches: both operands, rows padded to 16 bytes, B after A at 256 bytes
    assert q(BF16, 0, 0, 8191, 8191, 8191, base, 8191, base, 8191) == \
        rup(8191 * 8192 * 2, 256) + 8191 * 8192 * 2
    M, N, K = 4095, 2047, 3001          # stored shapes: A^T is K x M, B^T is N x K
    for ta in (0, 1):
        for tb in (0, 1):
            ar, ac = (K, M) if ta else (M, K)
            br, bc = (N, K) if tb else (K, N)
            want = rup(ar * rup(ac, 8) * 2, 256) + br * rup(bc, 8) * 2
            assert q(BF16, ta, tb, M, N, K, base, ac, base, bc) == want, (ta, tb)
    # in place: 4-byte-aligned rows with even outer extents (pair loads), and
    # 16-byte-aligned rows whatever the extents
    assert q(BF16, 0, 0, 8190, 8190, 8190, base, 8190, base, 8190) == 0
    assert q(BF16, 0, 0, 8191, 8191, 8191, base, 8192, base, 8192) == 0
    assert q(BF16, 1, 0, 8191, 8191, 8191, base, 8192, base, 8192) == 0
    # only the operand without 16-byte rows is copied: A at a 2-byte-aligned
    # address; B with an even pitch but an odd N along its rows
    assert q(BF16, 0, 0, 4096, 4096, 4096, base + 2, 4096, base, 4096) == 4096 * 4096 * 2
    assert q(BF16, 0, 0, 4096, 4095, 4096, base, 4096, base, 4098) == 4096 * 4096 * 2
    # the thresholds, one operand copied: M N / 8192 flops per copied byte of
    # an operand with 8192-element padded rows along N (B, outer-contiguous;
    # B^T, k-contiguous) or of A (k-contiguous)
    assert q(BF16, 0, 0, 57, 8191, 4096, base, 4096, base, 8191) == 4096 * 8192 * 2
    assert q(BF16, 0, 0, 56, 8191, 4096, base, 4096, base, 8191) == 0
    assert q(BF16, 0, 1, 161, 8191, 4096, base, 4096, base, 4097) == 8191 * 4096 * 2
    assert q(BF16, 0, 1, 159, 8191, 4096, base, 4096, base, 4097) == 0
    assert q(BF16, 0, 0, 8191, 161, 4096, base, 4097, base, 168) == rup(8191 * 4096 * 2, 256)
    assert q(BF16, 0, 0, 8191, 159, 4096, base, 4097, base, 168) == 0
    assert q(BF16, 1, 0, 8191, 57, 4096, base, 8191, base, 64) == rup(4096 * 8192 * 2, 256)
    assert q(BF16, 1, 0, 8191, 56, 4096, base, 8191, base, 64) == 0
    # both copied: 160 per byte of A plus 56 per byte of B
    assert q(BF16, 0, 0, 383, 383, 383, base, 383, base, 383) > 0
    assert q(BF16, 0, 0, 207, 207, 4096, base, 4097, base, 207) == 0
    assert q(BF16, 0, 0, 8191, 8191, 256, base, 257, base, 8191) > 0        # K = 256
    assert q(BF16, 0, 0, 8191, 8191, 255, base, 255, base, 8191) == 0       # K < 256: C-bound
    assert q(BF16, 0, 0, 320, 321, 256, base, 256, base, 321) == 0          # 313 per byte, < 2^26
    assert q(F32, 0, 0, 8191, 8191, 8191, base, 8191, base, 8191) == 0      # fp32: never
    assert q(BF16, 0, 0, 8191, 8191, 0, base, 1, base, 8191) == 0           # nothing to multiply
    # the arguments gemm_ex rejects
    bad = dg.GEMM_ERR_INVALID_ARG
    assert q(BF16, 0, 0, 10, 10, 10, base, 9, base, 10) == bad              # lda < K
    assert q(BF16, 0, 1, 10, 10, 10, base, 10, base, 9) == bad              # ldb < K for B^T
    assert q(BF16, 0, 0, 10, 10, 10, base + 1, 10, base, 10) == bad         # not element aligned
    assert q(BF16, 0, 0, 10, 10, 10, 0, 10, base, 10) == bad                # null A
    assert q(5, 0, 0, 10, 10, 10, base, 10, base, 10) == bad
    assert q(BF16, 2, 0, 10, 10, 10, base, 10, base, 10) == bad
    assert q(BF16, 0, 0, -1, 10, 10, base, 10, base, 10) == bad


def test_split_plan_with_aligned_rows_ignores_outer_parity():
    """With 16-byte-aligned rows the loads at the M and N edges run to the
    next 16 bytes, so every block takes the direct loads and the bf16 split
    plan of a shape with odd M or N is that of the padded shape."""
    BF16 = dg.GEMM_DTYPE_BF16
    for ta, tb in [(0, 0), (1, 0), (1, 1), (0, 1)]:
        for (M, N, K) in [(1535, 1535, 1536), (1023, 1021, 4096), (2001, 999, 3000)]:
            c = dg.gemm_select_config_ex(BF16, ta, tb, M, N, K)
            Mp, Np = -(-M // 8) * 8, -(-N // 8) * 8
            assert dg.gemm_select_config_ex(BF16, ta, tb, Mp, Np, K) == c
            assert dg.gemm_split_k_ex(BF16, c, ta, tb, M, N, K) == \
                dg.gemm_split_k_ex(BF16, c, ta, tb, Mp, Np, K), (ta, tb, M, N, K)


def test_config_table():
    for dtype, prefix in [(dg.GEMM_DTYPE_F32, "f32_"), (dg.GEMM_DTYPE_BF16, "bf16_")]:
        n = dg.gemm_num_configs(dtype)
        assert n >= 4
        for c in range(n):
            assert dg.gemm_config_name(dtype, c).startswith(prefix)
        assert dg.gemm_config_name(dtype, n) is None
        assert dg.gemm_config_name(dtype, -1) is None
    assert dg.gemm_num_configs(7) == dg.GEMM_ERR_INVALID_ARG


def _cfg_for(name):
    w = WORKLOADS[name]
    dtype = dg.GEMM_DTYPE_F32 if w.dtype == "f32" else dg.GEMM_DTYPE_BF16
    c = dg.gemm_select_config(dtype, w.M, w.N, w.K)
    return dtype, c, dg.gemm_config_name(dtype, c), dg.gemm_split_k(dtype, c, w.M, w.N, w.K)


def test_shape_classes_of_the_workloads():
    assert _cfg_for("fp32-4096")[2] == "f32_256x256_w4x2_s2"
    # 4097 x 4095: 256 blocks of 256 x 256 once the one-row remainder runs apart
    assert _cfg_for("fp32-rag")[2] == "f32_256x256_w4x2_s2"
    assert _cfg_for("bf16-8192")[2] == "bf16_256x256x64_w4x2_s2"
    assert _cfg_for("tall")[2] == "f32_128x64_w2x2_s2"
    dtype, c, name, splits = _cfg_for("im2col")
    assert name == "f32_64x256_w1x4_s2" and splits == 8
    # the same class for A^T . B (no two-stage kernel for that form)
    F32 = dg.GEMM_DTYPE_F32
    assert dg.gemm_config_name(F32, dg.gemm_select_config_ex(F32, 1, 0, 64, 16384, 61504)) == \
        "f32_64x256_w1x4_s3"
    # the convolution GEMMs with 32 output channels: 32-row blocks; the
    # filter gradient (B^T) with 256-byte k-contiguous rows and 16 slices
    F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16
    sel = lambda dt, tb, M, N, K: dg.gemm_config_name(dt, dg.gemm_select_config_ex(dt, 0, tb, M, N, K))
    assert sel(F32, 0, 32, 65536, 10976) == "f32_32x128_w1x4_s3"
    assert sel(F32, 1, 32, 10976, 65536) == "f32_32x128x64_w1x4_s2"
    assert sel(BF16, 0, 32, 65536, 10976) == "bf16_32x256x64_w1x4_s3"
    assert sel(BF16, 1, 32, 10976, 65536) == "bf16_32x256x128_w1x4_s2"
    assert sel(F32, 1, 64, 61504, 16384) == "f32_64x64x64_w2x2_s2"
    assert sel(BF16, 1, 64, 61504, 16384) == "bf16_64x64x64_w2x2_s4"
    c = dg.gemm_select_config_ex(F32, 0, 1, 32, 10976, 65536)
    assert dg.gemm_split_k_ex(F32, c, 0, 1, 32, 10976, 65536) == 16
    c = dg.gemm_select_config_ex(F32, 0, 1, 64, 61504, 16384)
    assert dg.gemm_split_k_ex(F32, c, 0, 1, 64, 61504, 16384) == 2   # 961 blocks already
    assert dg.gemm_split_k(F32, c, 64, 61504, 16384) == 1            # the same as A . B
    assert dg.gemm_split_k_ex(F32, c, 0, 2, 64, 61504, 16384) == dg.GEMM_ERR_INVALID_ARG
    for big in ("fp32-4096", "bf16-8192", "tall"):
        assert _cfg_for(big)[3] == 1
    # fp32 large class: 64x64 blocks in two stages where their grid fills
    # whole rounds better than three stages, three stages where those fill
    # whole rounds, and one-block entries only where their grid covers the chip
    for (M, N, K), name in [((2048, 2048, 2048), "f32_64x64_w2x2_s2"),
                            ((2560, 2560, 2560), "f32_64x64_w2x2_s2"),
                            ((3072, 3072, 3072), "f32_64x64_w2x2_s3"),
                            ((4096, 4096, 4096), "f32_256x256_w4x2_s2"),
                            ((2048, 4096, 2048), "f32_256x128_w4x2_s2")]:
        c = dg.gemm_select_config(F32, M, N, K)
        assert dg.gemm_config_name(F32, c) == name, (M, N, K)
        assert dg.gemm_split_k(F32, c, M, N, K) == 1
    # bf16 grids of exactly one 128x128 block per compute unit: three stages
    # (one resident block, nothing lost); more than one per unit: two stages
    for ta, tb in [(0, 0), (0, 1), (1, 0), (1, 1)]:
        assert dg.gemm_config_name(BF16, dg.gemm_select_config_ex(BF16, ta, tb, 2048, 2048, 2048)) \
            == "bf16_128x128x64_w2x2_s3"
        assert dg.gemm_config_name(BF16, dg.gemm_select_config_ex(BF16, ta, tb, 2560, 2560, 2560)) \
            == "bf16_128x128x64_w2x2_s2"
    # large bf16 with A k-contiguous (A . B, A . B^T): 64-deep k-tiles
    for tb in (0, 1):
        for M, N, K in [(8192, 8192, 8192), (4096, 4096, 4096)]:
            c = dg.gemm_select_config_ex(BF16, 0, tb, M, N, K)
            assert dg.gemm_config_name(BF16, c) == "bf16_256x256x64_w4x2_s2"
            assert dg.gemm_config_layouts(BF16, c) == (1 << 0) | (1 << 1)   # A . B and A . B^T
    for ta, tb in [(1, 0), (1, 1)]:
        assert dg.gemm_config_name(BF16, dg.gemm_select_config_ex(BF16, ta, tb, 8192, 8192, 8192)) \
            == "bf16_256x256x32_w4x2_s4"
    # 192 x 256 blocks (A . B and A . B^T) where 256 x 256 blocks would leave a
    # quarter or more of the chip idle, unsplit; not where 256 x 256 or
    # 128 x 128 blocks fill it better
    for tb in (0, 1):
        for (M, N, K), name in [((3072, 3072, 3072), "bf16_192x256x64_w2x4_s2"),
                                ((4608, 4608, 4608), "bf16_192x256x64_w2x4_s2"),
                                ((6144, 6144, 6144), "bf16_192x256x64_w2x4_s2"),
                                ((3072, 4096, 2048), "bf16_192x256x64_w2x4_s2"),
                                ((2560, 2560, 2560), "bf16_128x128x64_w2x2_s2"),
                                ((2304, 3072, 4096), "bf16_128x128x64_w2x2_s2"),
                                ((5120, 5120, 5120), "bf16_256x256x64_w4x2_s2")]:
            c = dg.gemm_select_config_ex(BF16, 0, tb, M, N, K)
            assert dg.gemm_config_name(BF16, c) == name, (M, N, K, tb)
            assert dg.gemm_split_k_ex(BF16, c, 0, tb, M, N, K) == 1, (M, N, K, tb)
    c = dg.gemm_select_config_ex(BF16, 0, 0, 3072, 3072, 3072)
    assert dg.gemm_config_layouts(BF16, c) == (1 << 0) | (1 << 1)
    assert dg.gemm_config_name(BF16, dg.gemm_select_config_ex(BF16, 1, 0, 3072, 3072, 3072)) \
        != "bf16_192x256x64_w2x4_s2"
    # bf16 mid-size and small products (256 compute units assumed off the GPU):
    # 128x128 blocks where they fill the chip or K is long (K-sliced when they
    # do not fill it), 64x64 blocks otherwise, four stages for small grids
    # with longer K; the 64-row blocks of M > 64 run unsplit
    for tb in (0, 1):
        for (M, N, K), name, splits in [
                ((1536, 1536, 1536), "bf16_64x64x64_w2x2_s2", 1),
                ((1024, 1024, 4096), "bf16_64x64x64_w2x2_s4", 1),
                ((768, 768, 2048), "bf16_64x64x64_w2x2_s4", 1),
                ((1000, 1000, 1000), "bf16_64x64x64_w2x2_s2", 1),
                ((1024, 1024, 8192), "bf16_128x128x64_w2x2_s2", 8),
                ((2000, 1000, 3000), "bf16_128x128x64_w2x2_s2", 3),
                ((1024, 4096, 1024), "bf16_128x128x64_w2x2_s3", 1)]:
            c = dg.gemm_select_config_ex(BF16, 0, tb, M, N, K)
            assert dg.gemm_config_name(BF16, c) == name, (M, N, K, tb)
            assert dg.gemm_split_k_ex(BF16, c, 0, tb, M, N, K) == splits, (M, N, K, tb)


def test_grid_fill_steers_the_large_class():
    """A 4096^2 output is 256 blocks of 256x256, one per compute unit; a
    6144^2 output would leave 3/4 of the second round idle with those blocks,
    so the 64x64 blocks (9216 of them, 3 per unit) win."""
    name = lambda M, N: dg.gemm_config_name(dg.GEMM_DTYPE_F32, dg.gemm_select_config(dg.GEMM_DTYPE_F32, M, N, 1024))
    assert name(4096, 4096) == "f32_256x256_w4x2_s2"
    assert name(8192, 8192) == "f32_256x256_w4x2_s2"
    assert name(6144, 6144) == "f32_64x64_w2x2_s3"


def test_split_plan_covers_k_with_nonempty_slices():
    for dtype in (dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16):
        for c in range(dg.gemm_num_configs(dtype)):
            for (M, N, K) in [(64, 16384, 61504), (64, 64, 100000), (1, 1, 1), (256, 256, 256),
                              (64, 256, 33), (50, 50, 4099)]:
                s = dg.gemm_split_k(dtype, c, M, N, K)
                assert 1 <= s <= max(1, K)


def test_invalid_arguments_rejected_before_any_device_call():
    p = 4096  # never dereferenced: every call below fails validation first
    bad = [
        (-1, 4, 4, p, 4, p, 4, p, 4),          # negative M
        (4, -1, 4, p, 4, p, 4, p, 4),          # negative N
        (4, 4, -1, p, 4, p, 4, p, 4),          # negative K
        (4, 4, 8, p, 7, p, 4, p, 4),           # lda < K
        (4, 4, 4, p, 4, p, 3, p, 4),           # ldb < N
        (4, 4, 4, p, 4, p, 4, p, 3),           # ldc < N
        (4, 4, 4, None, 4, p, 4, p, 4),        # null A
        (4, 4, 4, p, 4, None, 4, p, 4),        # null B
        (4, 4, 4, p, 4, p, 4, None, 4),        # null C
        (4, 4, 4, p + 2, 4, p, 4, p, 4),       # A not 4-byte aligned (fp32)
        (4, 4, 4, p, 4, p, 4, p + 1, 4),       # C not 4-byte aligned
        (1 << 31, 4, 4, p, 4, p, 4, p, 4),     # M beyond the supported range
    ]
    for args in bad:
        assert dg.gemm_f32(*args, None) == dg.GEMM_ERR_INVALID_ARG, args
    assert dg.gemm_bf16(4, 4, 4, p + 1, 4, p, 4, p, 4, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_f32_with_config(99, 0, 4, 4, 4, p, 4, p, 4, p, 4, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_f32_with_config(-1, 0, 4, 4, 4, p, 4, p, 4, p, 4, None) == dg.GEMM_ERR_INVALID_ARG


def test_gemm_ex_invalid_arguments_rejected_before_any_device_call():
    p = 4096
    F32, BF16, N_, T_ = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16, dg.GEMM_OP_N, dg.GEMM_OP_T
    ok = (F32, F32, N_, N_, 4, 6, 8, 1.0, p, 8, p, 6, 0.0, p, 6)

    def call(**kw):
        names = ["dt", "dtc", "ta", "tb", "M", "N", "K", "alpha", "A", "lda", "B", "ldb", "beta",
                 "C", "ldc"]
        args = dict(zip(names, ok))
        args.update(kw)
        return dg.gemm_ex(*[args[n] for n in names], None)

    bad = [
        dict(dt=2), dict(dtc=-1), dict(ta=2), dict(tb=-1),
        dict(M=-1), dict(K=1 << 31),
        dict(lda=7),                      # A as given: lda >= K = 8
        dict(ta=T_, lda=3),               # A transposed (K x M): lda >= M = 4
        dict(ldb=5),                      # B as given: ldb >= N = 6
        dict(tb=T_, ldb=7),               # B transposed (N x K): ldb >= K = 8
        dict(ldc=5),                      # ldc >= N
        dict(A=None), dict(B=None), dict(C=None),
        dict(C=p + 2),                    # fp32 C not 4-byte aligned
        dict(dtc=BF16, C=p + 1),          # bf16 C not 2-byte aligned
        dict(dt=BF16, A=p + 1),           # bf16 A not 2-byte aligned
    ]
    for kw in bad:
        assert call(**kw) == dg.GEMM_ERR_INVALID_ARG, kw
    # transposed leading dimensions that are valid for the stored shapes pass
    # validation; M == 0 then returns before any device call
    assert call(M=0, ta=T_, lda=1, C=None) == dg.GEMM_OK
    assert call(N=0, tb=T_, ldb=8, ldc=1, C=None) == dg.GEMM_OK
    # forced entries: out of range, or without kernels for the operand form
    assert dg.gemm_ex_with_config(99, 0, *ok, None) == dg.GEMM_ERR_INVALID_ARG
    for dtype in (F32, BF16):
        for c in range(dg.gemm_num_configs(dtype)):
            if not dg.gemm_config_layouts(dtype, c) & (1 << 3):
                args = (dtype, F32, T_, T_, 4, 6, 8, 1.0, p, 4, p, 8, 0.0, p, 6)
                assert dg.gemm_ex_with_config(c, 0, *args, None) == dg.GEMM_ERR_INVALID_ARG
                break


def test_layout_masks_cover_every_dispatched_entry():
    """The entry the dispatcher picks for an operand form has kernels for that
    form; the plain-product hook agrees with the general one at (N, N); every
    entry has kernels for some form."""
    for dtype in (dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16):
        for c in range(dg.gemm_num_configs(dtype)):
            assert dg.gemm_config_layouts(dtype, c) & 0xF
        assert dg.gemm_config_layouts(dtype, -1) == dg.GEMM_ERR_INVALID_ARG
        for M in (1, 20, 32, 33, 64, 65, 100, 1000, 2048, 4096, 8192, 65536):
            for N in (1, 33, 64, 65, 100, 1000, 1024, 2048, 4096, 16384):
                assert dg.gemm_select_config(dtype, M, N, 1024) == \
                    dg.gemm_select_config_ex(dtype, 0, 0, M, N, 1024)
                for ta in (0, 1):
                    for tb in (0, 1):
                        c = dg.gemm_select_config_ex(dtype, ta, tb, M, N, 1024)
                        assert dg.gemm_config_layouts(dtype, c) & (1 << (ta * 2 + tb)), \
                            (dtype, M, N, ta, tb)
        assert dg.gemm_select_config_ex(dtype, 2, 0, 4, 4, 4) == dg.GEMM_ERR_INVALID_ARG
        assert dg.gemm_select_config_ex(dtype, 0, 0, -1, 4, 4) == dg.GEMM_ERR_INVALID_ARG


def test_empty_output_is_a_no_op():
    # M == 0 or N == 0: nothing to compute, nothing launched, success.
    assert dg.gemm_f32(0, 5, 5, None, 5, None, 5, None, 5, None) == dg.GEMM_OK
    assert dg.gemm_bf16(5, 0, 5, None, 5, None, 1, None, 1, None) == dg.GEMM_OK


def test_missing_library_raises(tmp_path):
    import importlib
    mod = importlib.import_module("dense_gemm_03_amd")
    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(RuntimeError, match="no CPU fallback"):
            mod.load_library(str(tmp_path / "absent.so"))
    finally:
        mod._lib = saved


def test_conv_host_logic_and_invalid_arguments():
    """Output sizes, workspace sizes and argument checks of the convolution
    entry points; every invalid call fails before any device call."""
    P = dg.conv2d_params
    assert dg.conv2d_output_size(P(1, 64, 128, 128, 64, 31, 31, (15, 15))) == (0, 128, 128)
    assert dg.conv2d_output_size(P(2, 3, 10, 9, 4, 3, 2, (1, 0), (2, 3), (1, 2)))[1:] == (5, 3)
    # workspace: C_in R S rows of round_up(P Q, 8) elements
    assert dg.conv2d_workspace_size(dg.GEMM_DTYPE_F32, P(1, 64, 128, 128, 64, 31, 31, (15, 15))) \
        == 61504 * 16384 * 4
    assert dg.conv2d_workspace_size(dg.GEMM_DTYPE_BF16, P(1, 2, 5, 5, 1, 3, 3)) == 18 * 16 * 2
    bad = [P(1, 0, 8, 8, 1, 3, 3), P(1, 1, 8, 8, 1, 3, 3, (-1, 0)), P(1, 1, 8, 8, 1, 3, 3, (0, 0), (0, 1)),
           P(1, 1, 8, 8, 1, 3, 3, (0, 0), (1, 1), (1, 0)), P(1, 1, 2, 8, 1, 3, 3),
           P(-1, 1, 8, 8, 1, 3, 3), P(1, 1, 1 << 31, 8, 1, 3, 3), P(1, 1 << 16, 8, 8, 1, 1 << 8, 1 << 8)]
    for params in bad:
        assert dg.conv2d_output_size(params)[0] == dg.GEMM_ERR_INVALID_ARG
        assert dg.conv2d_workspace_size(dg.GEMM_DTYPE_F32, params) == dg.GEMM_ERR_INVALID_ARG
    ok = P(2, 3, 10, 9, 4, 3, 2, (1, 0))
    assert dg.conv2d_output_size(ok) == (0, 10, 8)
    need = dg.conv2d_workspace_size(dg.GEMM_DTYPE_F32, ok)
    p = 4096
    F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16
    assert dg.conv2d_workspace_size(5, ok) == dg.GEMM_ERR_INVALID_ARG
    calls = [
        lambda: dg.conv2d_fwd(F32, F32, bad[0], p, p, p, p, need),
        lambda: dg.conv2d_fwd(7, F32, ok, p, p, p, p, need),
        lambda: dg.conv2d_fwd(F32, 7, ok, p, p, p, p, need),
        lambda: dg.conv2d_fwd(F32, F32, ok, None, p, p, p, need),
        lambda: dg.conv2d_fwd(F32, F32, ok, p, None, p, p, need),
        lambda: dg.conv2d_fwd(F32, F32, ok, p, p, None, p, need),
        lambda: dg.conv2d_fwd(F32, F32, ok, p, p, p, None, need),
        lambda: dg.conv2d_fwd(F32, F32, ok, p, p, p, p, need - 1),      # workspace too small
        lambda: dg.conv2d_fwd(F32, F32, ok, p, p, p, p + 8, need),      # workspace not 16-aligned
        lambda: dg.conv2d_fwd(F32, F32, ok, p + 2, p, p, p, need),      # x misaligned
        lambda: dg.conv2d_fwd(BF16, BF16, ok, p, p, p + 1, p, need),    # bf16 y misaligned
        lambda: dg.conv2d_bwd_weight(F32, ok, p, p, p + 2, p, need),    # dw misaligned
        lambda: dg.conv2d_bwd_weight(F32, ok, None, p, p, p, need),
        lambda: dg.conv2d_bwd_weight(F32, ok, p, p, p, p, need - 4),
        lambda: dg.conv2d_im2col(F32, ok, 2, p, p, 80),                 # image out of range
        lambda: dg.conv2d_im2col(F32, ok, -1, p, p, 80),
        lambda: dg.conv2d_im2col(F32, ok, 0, p, p, 79),                 # ld_cols < P Q = 80
        lambda: dg.conv2d_im2col(F32, ok, 0, None, p, 80),
        lambda: dg.conv2d_im2col(F32, ok, 0, p, p + 2, 80),             # cols misaligned
    ]
    for t, call in enumerate(calls):
        assert call() == dg.GEMM_ERR_INVALID_ARG, t
    # implicit-GEMM forms: same checks, no workspace; one image must span < 2 GiB
    assert dg.conv2d_fwd_implicit(F32, F32, bad[0], p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_fwd_implicit(F32, F32, ok, None, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_fwd_implicit(F32, 9, ok, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_bwd_weight_implicit(F32, ok, p, p, p + 2) == dg.GEMM_ERR_INVALID_ARG
    huge = P(1, 2, 1 << 15, 1 << 14, 1, 3, 3)       # 2 x 2^29 fp32 elements = 4 GiB per image
    assert dg.conv2d_output_size(huge)[0] == dg.GEMM_OK
    assert dg.conv2d_fwd_implicit(F32, F32, huge, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_bwd_weight_implicit(BF16, huge, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    # address generation: unknown forms are rejected; the table form needs its
    # y and x terms within signed 16 bits
    A, T, PD = dg.CONV_ADDR_ANALYTIC, dg.CONV_ADDR_TABLE, dg.CONV_ADDR_PADDED
    assert dg.conv2d_fwd_implicit_ex(F32, F32, ok, 5, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_fwd_implicit_ex(F32, F32, ok, -1, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_bwd_weight_implicit_ex(F32, ok, 7, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    wide = P(1, 1, 40001, 8, 1, 3, 1, (0, 0), (1, 1), (20000, 1))   # (R-1) dh = 40000
    assert dg.conv2d_output_size(wide)[0] == dg.GEMM_OK
    assert dg.conv2d_fwd_implicit_ex(F32, F32, wide, T, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    tall = P(1, 1, 70000, 4, 1, 1, 1)                              # last p sh - ph = 69999
    assert dg.conv2d_bwd_weight_implicit_ex(F32, tall, T, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_fwd_implicit_ex(F32, F32, bad[0], A, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    # the padded form needs the padded image below 2 GiB: this image is just
    # under it (2^31 - 2^19 bytes), its copy with 2-wide zero borders is not
    edge = P(1, 1, 1 << 14, (1 << 15) - 8, 1, 5, 5, (2, 2))
    assert dg.conv2d_output_size(edge)[0] == dg.GEMM_OK
    assert dg.conv2d_fwd_implicit_ex(F32, F32, edge, PD, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    # the window form reads the same copy
    assert dg.conv2d_fwd_implicit_ex(F32, F32, edge, dg.CONV_ADDR_WINDOW, p, p, p) == \
        dg.GEMM_ERR_INVALID_ARG
    assert dg.conv2d_bwd_weight_implicit_ex(F32, edge, PD, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    # an empty batch: nothing to compute for the forward
    assert dg.conv2d_fwd(F32, F32, P(0, 3, 10, 9, 4, 3, 2), None, None, None, None, 0) == dg.GEMM_OK


def test_convnd_host_logic_and_invalid_arguments():
    """Output and workspace sizes of the N-D entry points, the 2-D case equal
    to the conv2d calls', and argument checks that fail before any device
    call."""
    N = dg.convnd_params
    p3 = N(1, 32, 32, (16, 64, 64), (7, 7, 7), (3, 3, 3))
    assert dg.convnd_output_size(p3) == (0, (16, 64, 64))
    assert dg.convnd_workspace_size(dg.GEMM_DTYPE_F32, p3) == 32 * 343 * 65536 * 4
    p4 = N(2, 16, 32, (6, 6, 24, 24), (3, 3, 5, 5), (1, 1, 2, 2))
    assert dg.convnd_output_size(p4) == (0, (6, 6, 24, 24))
    p1 = N(1, 2, 3, (37,), (5,), (2,), (2,), (1,))
    assert dg.convnd_output_size(p1) == (0, (19,))
    # rows C_in prod(K), columns round_up(prod(O), 8)
    assert dg.convnd_workspace_size(dg.GEMM_DTYPE_BF16, p1) == 2 * 5 * 24 * 2
    # D = 2 gives the conv2d numbers
    for args in [(2, 3, 10, 9, 4, 3, 2, (1, 0), (2, 3), (1, 2)), (1, 64, 128, 128, 64, 31, 31, (15, 15))]:
        b, ci, h, w, co, r, s_ = args[:7]
        pad, stride, dil = (list(args[7:]) + [(0, 0), (1, 1), (1, 1)][len(args) - 7:])[:3]
        p2 = dg.conv2d_params(*args)
        pn = N(b, ci, co, (h, w), (r, s_), pad, stride, dil)
        rc, P, Q = dg.conv2d_output_size(p2)
        assert dg.convnd_output_size(pn) == (rc, (P, Q))
        for dt in (dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16):
            assert dg.convnd_workspace_size(dt, pn) == dg.conv2d_workspace_size(dt, p2)
    bad = [N(1, 0, 1, (8,), (3,)), N(1, 1, 1, (8, 8), (9, 1)), N(1, 1, 1, (8,), (3,), (-1,)),
           N(1, 1, 1, (8,), (3,), (0,), (0,)), N(1, 1, 1, (8,), (3,), (0,), (1,), (0,)),
           N(-1, 1, 1, (8,), (3,)), N(1, 1, 1, (1 << 16, 1 << 15), (1, 1)),  # 2^31 per channel
           N(1, 1 << 16, 1, (32, 32, 32), (32, 32, 32))]                     # C_in prod(K) = 2^31
    for params in bad:
        assert dg.convnd_output_size(params)[0] == dg.GEMM_ERR_INVALID_ARG, params.ndim
        assert dg.convnd_workspace_size(dg.GEMM_DTYPE_F32, params) == dg.GEMM_ERR_INVALID_ARG
    for nd in (0, 5, -1):
        q = N(1, 1, 1, (8,), (3,))
        q.ndim = nd
        assert dg.convnd_output_size(q)[0] == dg.GEMM_ERR_INVALID_ARG
        assert dg.convnd_workspace_size(dg.GEMM_DTYPE_F32, q) == dg.GEMM_ERR_INVALID_ARG
    assert dg.load_library().convnd_output_size(None, None) == dg.GEMM_ERR_INVALID_ARG
    ok = N(2, 3, 4, (5, 6, 7), (3, 2, 3), (1, 0, 1))
    need = dg.convnd_workspace_size(dg.GEMM_DTYPE_F32, ok)
    vo = 5 * 5 * 7
    p = 4096
    F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16
    assert dg.convnd_workspace_size(5, ok) == dg.GEMM_ERR_INVALID_ARG
    calls = [
        lambda: dg.convnd_fwd(F32, F32, bad[0], p, p, p, p, need),
        lambda: dg.convnd_fwd(7, F32, ok, p, p, p, p, need),
        lambda: dg.convnd_fwd(F32, 7, ok, p, p, p, p, need),
        lambda: dg.convnd_fwd(F32, F32, ok, None, p, p, p, need),
        lambda: dg.convnd_fwd(F32, F32, ok, p, p, p, p, need - 1),
        lambda: dg.convnd_fwd(F32, F32, ok, p, p, p, p + 8, need),
        lambda: dg.convnd_fwd(BF16, BF16, ok, p, p, p + 1, p, need),
        lambda: dg.convnd_bwd_weight(F32, ok, p, p, p + 2, p, need),
        lambda: dg.convnd_bwd_weight(F32, ok, p, None, p, p, need),
        lambda: dg.convnd_im2col(F32, ok, 2, p, p, vo),
        lambda: dg.convnd_im2col(F32, ok, 0, p, p, vo - 1),
        lambda: dg.convnd_im2col(BF16, ok, 0, p + 1, p, vo),
    ]
    for t, call in enumerate(calls):
        assert call() == dg.GEMM_ERR_INVALID_ARG, t
    assert dg.convnd_fwd(F32, F32, N(0, 3, 4, (5,), (3,)), None, None, None, None, 0) == dg.GEMM_OK
    # implicit forms: one to four dimensions, one image below 2 GiB
    assert dg.convnd_fwd_implicit(F32, F32, p4, p, p, p + 2) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_bwd_weight_implicit(F32, p4, p, p + 1, p) == dg.GEMM_ERR_INVALID_ARG
    big4 = N(1, 4, 1, (2, 256, 512, 512), (1, 1, 1, 1))   # 4 x 2^27 fp32 elements: 2 GiB
    assert dg.convnd_fwd_implicit(F32, F32, big4, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_bwd_weight_implicit(F32, big4, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_fwd_implicit(F32, F32, bad[0], p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_fwd_implicit(F32, F32, ok, None, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_bwd_weight_implicit(F32, ok, p, p, p + 2) == dg.GEMM_ERR_INVALID_ARG
    big = N(1, 4, 1, (512, 512, 512), (1, 1, 1))      # 4 x 2^27 fp32 elements: 2 GiB
    assert dg.convnd_fwd_implicit(F32, F32, big, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    assert dg.convnd_fwd_implicit(F32, F32, N(0, 3, 4, (5,), (3,)), None, None, None) == dg.GEMM_OK
    # addressing: analytic, padded or the default; the table form is 2-D only
    for mode in (dg.CONV_ADDR_TABLE, 5, -1):
        assert dg.convnd_fwd_implicit_ex(F32, F32, ok, mode, p, p, p) == dg.GEMM_ERR_INVALID_ARG
        assert dg.convnd_bwd_weight_implicit_ex(F32, ok, mode, p, p, p) == dg.GEMM_ERR_INVALID_ARG
    # an image just under 2 GiB whose zero-bordered copy is not
    edge = N(1, 1, 1, (8, 1 << 12, (1 << 14) - 8), (3, 3, 3), (1, 1, 1))
    assert dg.convnd_output_size(edge)[0] == dg.GEMM_OK
    assert dg.convnd_fwd_implicit_ex(F32, F32, edge, dg.CONV_ADDR_PADDED, p, p, p) == \
        dg.GEMM_ERR_INVALID_ARG
