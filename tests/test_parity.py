"""GPU parity: the HIP kernels against the oracle, through the C ABI.

Integer-valued operands make every partial sum exact, so those results must
equal the oracle bit for bit whatever the summation order; they catch dropped
or repeated k terms, misplaced fragments, LDS races and edge bugs.  Random
operands check the tolerance max|C - C_ref| / S <= 1e-5 (fp32) and 4e-3 (bf16
inputs).  Every configuration of the tile table runs, with 16-byte aligned and
unaligned leading dimensions, at shapes that span several tiles and end in
ragged tails.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_03_amd as dg
from dense_gemm_03_amd import workloads as wl
from tests.gpu_util import check_close, check_exact, log, run, to_device

pytestmark = pytest.mark.gpu

F32, BF16 = dg.GEMM_DTYPE_F32, dg.GEMM_DTYPE_BF16


def _configs(dtype):
    """Entries with kernels for the plain product A . B (entries built only
    for A . B^T are covered by tests/test_variants.py)."""
    return [c for c in range(dg.gemm_num_configs(dtype)) if dg.gemm_config_layouts(dtype, c) & 1]


def _ints(shape, seed, bf16):
    return wl.small_int_bf16_bits(shape, seed) if bf16 else wl.small_int_f32(shape, seed)


SHAPES = [
    (1, 1, 1),
    (7, 5, 3),
    (64, 64, 64),
    (256, 256, 256),
    (300, 200, 100),
    (129, 257, 71),
    (33, 300, 1000),
    (520, 72, 260),
]


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_exact_integers_every_config(bf16):
    dtype = BF16 if bf16 else F32
    for cfg in _configs(dtype):
        name = dg.gemm_config_name(dtype, cfg)
        for t, (M, N, K) in enumerate(SHAPES):
            A = _ints((M, K), 10 + t, bf16)
            B = _ints((K, N), 20 + t, bf16)
            log("%s M=%d N=%d K=%d aligned" % (name, M, N, K))
            C = run(A, B, cfg=cfg).cpu().numpy()
            check_exact(C, A, B, "%s %dx%dx%d" % (name, M, N, K))
            # odd leading dimensions (element-wise load path), padding holds NaN
            nan = wl.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] if bf16 else np.nan
            log("%s M=%d N=%d K=%d unaligned" % (name, M, N, K))
            C = run(A, B, cfg=cfg, pad_a=1, pad_b=3, fill=nan).cpu().numpy()
            check_exact(C, A, B, "%s %dx%dx%d unaligned" % (name, M, N, K))


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_one_hot_probes_place_every_fragment(bf16):
    """A = e_i e_k^T copies row k of B into row i of C and nothing else: pins
    the lane layout of MFMA operands and accumulators, for positions in every
    32-row fragment of a 256-row block and at tile edges."""
    dtype = BF16 if bf16 else F32
    M, N, K = 260, 130, 97
    B = _ints((K, N), 5, bf16)
    one = wl.f32_to_bf16_bits(np.array([1.0], np.float32))[0] if bf16 else np.float32(1)
    for cfg in _configs(dtype):
        for i, k in [(0, 0), (31, 1), (32, 63), (77, 64), (128, 5), (255, 96), (259, 50)]:
            A = np.zeros((M, K), dtype=B.dtype)
            A[i, k] = one
            C = run(A, B, cfg=cfg).cpu().numpy()
            check_exact(C, A, B, "%s one-hot (%d,%d)" % (dg.gemm_config_name(dtype, cfg), i, k))


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_random_within_tolerance_every_config(bf16):
    dtype = BF16 if bf16 else F32
    M, N, K = 333, 301, 517
    if bf16:
        A, B = wl.normal_bf16_bits((M, K), 1), wl.normal_bf16_bits((K, N), 2)
    else:
        A, B = wl.uniform_f32((M, K), 1), wl.uniform_f32((K, N), 2)
    for cfg in _configs(dtype):
        name = dg.gemm_config_name(dtype, cfg)
        check_close(run(A, B, cfg=cfg).cpu().numpy(), A, B, name)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_forced_split_k(bf16):
    """Split-K with a deterministic reduce: exact on integers, within tolerance
    on random values, for several slice counts including uneven ones."""
    dtype = BF16 if bf16 else F32
    M, N, K = 70, 520, 3001
    A, B = _ints((M, K), 3, bf16), _ints((K, N), 4, bf16)
    for cfg in _configs(dtype):
        for s in (2, 3, 7):
            C = run(A, B, cfg=cfg, split_k=s).cpu().numpy()
            check_exact(C, A, B, "%s split %d" % (dg.gemm_config_name(dtype, cfg), s))
    if bf16:
        A, B = wl.normal_bf16_bits((M, K), 5), wl.normal_bf16_bits((K, N), 6)
    else:
        A, B = wl.uniform_f32((M, K), 5), wl.uniform_f32((K, N), 6)
    check_close(run(A, B, cfg=0, split_k=5).cpu().numpy(), A, B, "split 5 random")


def test_guard_bands_untouched():
    """C inside a larger NaN-filled buffer (ldc > N, rows above and below):
    only the M x N window is written."""
    import torch
    for bf16 in (False, True):
        M, N, K = 131, 77, 45
        A, B = _ints((M, K), 7, bf16), _ints((K, N), 8, bf16)
        big = torch.full((M + 2, N + 9), float("nan"), dtype=torch.float32, device="cuda:0")
        out = big[1:M + 1, :N]
        run(A, B, out=out)
        host = big.cpu().numpy()
        check_exact(host[1:M + 1, :N], A, B, "guarded window")
        assert np.all(np.isnan(host[0])) and np.all(np.isnan(host[M + 1]))
        assert np.all(np.isnan(host[1:M + 1, N:]))


def test_k_zero_fills_zeros_and_empty_is_noop():
    import torch
    C = torch.full((5, 7), float("nan"), device="cuda:0")
    A = torch.empty((5, 0), device="cuda:0")
    B = torch.empty((0, 7), device="cuda:0")
    dg.gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    E = torch.full((0, 7), float("nan"), device="cuda:0")
    dg.gemm(torch.empty((0, 3), device="cuda:0"), torch.ones((3, 7), device="cuda:0"), out=E)


def test_nan_propagates_only_where_it_belongs():
    """A NaN in A[i][k] makes row i of C NaN (IEEE) and nothing else; padding
    beyond K is never multiplied in."""
    M, N, K = 200, 150, 90
    A = wl.small_int_f32((M, K), 1)
    B = wl.small_int_f32((K, N), 2)
    A[17, 33] = np.nan
    C = run(A, B).cpu().numpy()
    assert np.all(np.isnan(C[17]))
    rest = np.delete(C, 17, axis=0)
    assert np.all(np.isfinite(rest))


def test_deterministic_repeats():
    import torch
    for (M, N, K, bf16) in [(1000, 1000, 1000, False), (64, 4096, 20000, False), (512, 512, 512, True)]:
        if bf16:
            A, B = wl.normal_bf16_bits((M, K), 1), wl.normal_bf16_bits((K, N), 2)
        else:
            A, B = wl.uniform_f32((M, K), 1), wl.uniform_f32((K, N), 2)
        Ad, Bd = to_device(A), to_device(B)
        outs = [dg.gemm(Ad, Bd) for _ in range(3)]
        torch.cuda.synchronize()
        assert all(torch.equal(outs[0], o) for o in outs[1:]), (M, N, K)


def test_transpose_invariant_on_gpu():
    """(A.B)^T == B^T.A^T bitwise for integer operands."""
    for bf16 in (False, True):
        A, B = _ints((150, 230), 1, bf16), _ints((230, 90), 2, bf16)
        C = run(A, B).cpu().numpy()
        Ct = run(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T)).cpu().numpy()
        assert np.array_equal(C.T, Ct)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
def test_leading_dimensions_beyond_32_bit_tile_offsets(bf16):
    """Leading dimensions so large that a tile's byte offsets from its origin
    exceed 32 bits (A rows 16 MiB + 32 bytes apart, C likewise): the kernels
    take their 64-bit element-wise path.  The padding holds NaN and must be
    neither read (C finite and exact) nor written."""
    import torch
    M, N, K = 300, 200, 100
    ld = (1 << 22) + 8                                   # elements; 256 rows x ld x 4 B > 2^32
    dt = torch.bfloat16 if bf16 else torch.float32
    A, B = _ints((M, K), 91, bf16), _ints((K, N), 92, bf16)
    Abuf = torch.full((M, ld), float("nan"), dtype=dt, device="cuda:0")
    Abuf[:, :K] = to_device(A)
    Cbuf = torch.full((M, ld), float("nan"), dtype=torch.float32, device="cuda:0")
    C = Cbuf[:, :N]
    dg.gemm(Abuf[:, :K], to_device(B), out=C)
    torch.cuda.synchronize()
    check_exact(C.cpu().numpy(), A, B, "lda = ldc = %d" % ld)
    assert bool(torch.isnan(Cbuf[:, N:N + 64]).all()) and bool(torch.isnan(Cbuf[:, -8:]).all())
    del Abuf, Cbuf
    torch.cuda.empty_cache()
