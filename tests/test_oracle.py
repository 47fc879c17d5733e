"""The oracle against its pins (CPU only).

Every pin in ``oracle_pins`` runs against the C oracle through both operand
encodings (fp32 and bf16 bit patterns).  Mutants with planted mistakes (a
dropped k term, a transposed operand, a flipped sign, an index off by one, a
wrong tolerance scale) must each fail at least one pin, which shows that the
pins can tell a wrong oracle from a right one.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_03_amd import workloads
from tests import oracle_pins as pins


# ---------------------------------------------------------------- adapters --

def _f32_gemm(A, B):
    A32 = np.ascontiguousarray(A, dtype=np.float32)
    B32 = np.ascontiguousarray(B, dtype=np.float32)
    assert np.array_equal(A32.astype(np.float64), A) and np.array_equal(B32.astype(np.float64), B), \
        "test value not representable in fp32"
    return oracle.gemm_f32(A32, B32, threads=3)


_f32_gemm.quantize = lambda x: np.asarray(x, dtype=np.float32).astype(np.float64)


def _bf16_quant(x):
    bits = workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return oracle.bf16_bits_to_f64(bits).reshape(np.shape(x))


def _to_bf16_bits(x):
    bits = workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)).reshape(np.shape(x))
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x), "test value not representable in bf16"
    return bits


def _bf16_gemm(A, B):
    return oracle.gemm_bf16(_to_bf16_bits(A), _to_bf16_bits(B), threads=2)


_bf16_gemm.quantize = _bf16_quant


ENCODINGS = {"f32": _f32_gemm, "bf16": _bf16_gemm}


# ------------------------------------------------------------------- pins --

@pytest.mark.parametrize("enc", sorted(ENCODINGS))
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: getattr(p, "__name__", "bruteforce5"))
def test_pin(enc, pin):
    pin(ENCODINGS[enc])


def test_bruteforce_all_shapes_to_8():
    """Every (m, n, k) in {1..8}^3 with small integers, exact."""
    pins.pin_bruteforce_integers(_f32_gemm, max_dim=8)


def test_bruteforce_dyadic_exact():
    """Dyadic rationals j/2^p with few bits: the fp64 sums stay exact, so the
    oracle equals the rational result bit for bit."""
    rng = np.random.default_rng(17)
    for m, n, k in [(3, 4, 5), (8, 1, 8), (1, 8, 7), (6, 6, 6)]:
        A = rng.integers(-64, 65, size=(m, k)) / 32.0
        B = rng.integers(-64, 65, size=(k, n)) / 16.0
        C, S = _f32_gemm(A, B)
        Ce, Se = pins.exact_product(A, B)
        for i in range(m):
            for j in range(n):
                assert pins.Fraction(float(C[i, j])) == Ce[i][j]
                assert pins.Fraction(float(S[i, j])) == Se[i][j]


def test_bruteforce_reals_within_fp64_bound():
    shapes = [(1, 1, 1), (2, 3, 4), (5, 7, 8), (8, 8, 8), (3, 2, 64)]
    pins.pin_bruteforce_reals(
        _f32_gemm, lambda rng, s: rng.uniform(-1, 1, size=s).astype(np.float32).astype(np.float64), shapes)
    pins.pin_bruteforce_reals(
        _bf16_gemm, lambda rng, s: _bf16_quant(rng.standard_normal(size=s)), shapes)


# ---------------------------------------------------------------- mutants --

def _mutant(name):
    """An oracle with one planted mistake, built around the real one."""
    def drop_last_k(A, B):
        return _f32_gemm(A[:, :-1], B[:-1, :]) if A.shape[1] > 1 else (
            np.zeros((A.shape[0], B.shape[1])), np.zeros((A.shape[0], B.shape[1])))

    def transpose_b(A, B):
        if B.shape[0] == B.shape[1]:
            return _f32_gemm(A, np.ascontiguousarray(B.T))
        return _f32_gemm(A, B)  # only square B can be mis-read this way

    def flip_sign(A, B):
        C, S = _f32_gemm(A, B)
        return -C if A.shape[1] > 2 else C, S

    def k_off_by_one(A, B):
        # pairs A[:, k] with B[k+1, :] (cyclically)
        return _f32_gemm(A, np.ascontiguousarray(np.roll(B, -1, axis=0)))

    def s_signed(A, B):
        C, _ = _f32_gemm(A, B)
        return C, C  # tolerance scale computed without absolute values

    def rows_swapped(A, B):
        C, S = _f32_gemm(A, B)
        if C.shape[0] > 1:
            C = C.copy()
            C[[0, -1]] = C[[-1, 0]]
        return C, S

    fns = {f.__name__: f for f in [drop_last_k, transpose_b, flip_sign, k_off_by_one, s_signed,
                                   rows_swapped]}
    fn = fns[name]
    fn.quantize = _f32_gemm.quantize
    return fn


@pytest.mark.parametrize("name", ["drop_last_k", "transpose_b", "flip_sign", "k_off_by_one",
                                  "s_signed", "rows_swapped"])
def test_pins_catch_planted_mistake(name):
    mutant = _mutant(name)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except pins.PinFailure:
            failed.append(pin)
    assert failed, "mutant %s passed every pin" % name


# ----------------------------------------------------- interface and edges --

def test_bf16_decode_known_patterns():
    """Known bf16 encodings (IEEE binary32 upper halves), decoded through a
    1x1x1 product with 1.0 (0x3F80)."""
    cases = {
        0x3F80: 1.0, 0x4000: 2.0, 0xBF80: -1.0, 0x3F81: 1.0 + 2.0 ** -7,
        0x0001: 2.0 ** -133, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x8000: -0.0,
        0x3E80: 0.25, 0xC2F6: -123.0,
    }
    one = np.array([[0x3F80]], dtype=np.uint16)
    for bits, value in cases.items():
        C, S = oracle.gemm_bf16(np.array([[bits]], dtype=np.uint16), one)
        assert C[0, 0] == value and S[0, 0] == abs(value), hex(bits)


def test_k_zero_gives_zero_and_empty_shapes():
    A = np.zeros((3, 0), dtype=np.float32)
    B = np.zeros((0, 4), dtype=np.float32)
    C, S = oracle.gemm_f32(A, B)
    assert C.shape == (3, 4) and np.all(C == 0) and np.all(S == 0)
    C, S = oracle.gemm_f32(np.zeros((0, 5), np.float32), np.ones((5, 2), np.float32))
    assert C.shape == (0, 2)
    C, S = oracle.gemm_f32(np.ones((2, 5), np.float32), np.ones((5, 0), np.float32))
    assert C.shape == (2, 0)


def test_leading_dimensions_ignore_padding():
    """Operands passed as row-strided views: the padding (NaN) is never read."""
    Abig = np.full((17, 40), np.nan, dtype=np.float32)
    Bbig = np.full((29, 50), np.nan, dtype=np.float32)
    A = workloads.uniform_f32((17, 29), 1)
    B = workloads.uniform_f32((29, 33), 2)
    Abig[:, :29] = A
    Bbig[:, :33] = B
    C1, S1 = oracle.gemm_f32(A, B)
    C2, S2 = oracle.gemm_f32(Abig[:, :29], Bbig[:, :33])
    assert np.array_equal(C1, C2) and np.array_equal(S1, S2)


def test_threads_do_not_change_sums():
    A = workloads.uniform_f32((61, 70), 5)
    B = workloads.uniform_f32((70, 45), 6)
    C1, S1 = oracle.gemm_f32(A, B, threads=1)
    C7, S7 = oracle.gemm_f32(A, B, threads=7)
    C99, _ = oracle.gemm_f32(A, B, threads=99)
    assert np.array_equal(C1, C7) and np.array_equal(S1, S7) and np.array_equal(C1, C99)


def test_against_numpy_float64_within_bound():
    """Library cross-check: numpy's float64 product of the same (exactly
    widened) operands differs from the oracle by at most the sum of both
    summation error bounds, 2 * (K - 1) * 2^-53 * S."""
    for (m, n, k, seed) in [(64, 96, 300, 1), (5, 700, 1000, 2)]:
        A = workloads.uniform_f32((m, k), seed)
        B = workloads.uniform_f32((k, n), seed + 1)
        C, S = oracle.gemm_f32(A, B)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        assert np.all(np.abs(C - ref) <= 2 * (k - 1) * 2.0 ** -53 * S)


def test_entries_match_full_product_bitwise():
    """The single-entry path sums in the same k order as the full product."""
    A = workloads.uniform_f32((50, 77), 8)
    B = workloads.uniform_f32((77, 31), 9)
    C, S = oracle.gemm_f32(A, B)
    I, J = workloads.sample_positions(50, 31, 40, 3)
    c, s = oracle.entries_f32(A, B, I, J)
    assert np.array_equal(c, C[I, J]) and np.array_equal(s, S[I, J])
    Ab = workloads.normal_bf16_bits((20, 64), 1)
    Bb = workloads.normal_bf16_bits((64, 24), 2)
    C, S = oracle.gemm_bf16(Ab, Bb)
    I, J = workloads.sample_positions(20, 24, 30, 4)
    c, s = oracle.entries_bf16(Ab, Bb, I, J)
    assert np.array_equal(c, C[I, J]) and np.array_equal(s, S[I, J])


def test_invalid_arguments_rejected():
    lib = oracle._load()
    A = np.ones((2, 2), np.float32)
    out = np.zeros((2, 2))
    p = A.ctypes.data
    o = out.ctypes.data
    assert lib.oracle_gemm_f32(-1, 2, 2, p, 2, p, 2, o, 2, o, 2, 1) == -1
    assert lib.oracle_gemm_f32(2, 2, 2, p, 1, p, 2, o, 2, o, 2, 1) == -1  # lda < K
    assert lib.oracle_gemm_f32(2, 2, 2, p, 2, p, 1, o, 2, o, 2, 1) == -1  # ldb < N
    assert lib.oracle_gemm_f32(2, 2, 2, None, 2, p, 2, o, 2, o, 2, 1) == -1
    I = np.array([5], np.int64)
    J = np.array([0], np.int64)
    c = np.zeros(1)
    assert lib.oracle_entries_f32(2, 2, 2, p, 2, p, 2, 1, I.ctypes.data, J.ctypes.data,
                                  c.ctypes.data, c.ctypes.data) == -1
    with pytest.raises(ValueError):
        oracle.gemm_f32(np.ones((2, 3), np.float32), np.ones((2, 3), np.float32))



def test_error_ratio_checker():
    C_ref = np.array([[1.0, 0.0], [2.0, -3.0]])
    S = np.array([[2.0, 0.0], [4.0, 6.0]])
    r, z = oracle.max_error_ratio(C_ref + np.array([[0.002, 0.0], [0.0, 0.0]]), C_ref, S)
    assert abs(r - 0.001) < 1e-15 and z
    r, z = oracle.max_error_ratio(C_ref + np.array([[0.0, 1e-30], [0.0, 0.0]]), C_ref, S)
    assert not z
    r, _ = oracle.max_error_ratio(np.array([[np.nan, 0.0], [2.0, -3.0]]), C_ref, S)
    assert r == float("inf")


# ------------------------------------------------------------ input recipe --

def test_bf16_rounding_matches_torch():
    """The generator's float32 -> bf16 rounding (nearest, ties to even) agrees
    with torch's conversion, including exact ties."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    # exact halfway cases (low 16 bits = 0x8000), both signs, odd and even upper halves
    hi = np.concatenate([np.arange(0x3F00, 0x3F80, dtype=np.uint32), np.arange(0xBF00, 0xBF80, dtype=np.uint32)])
    ties = ((hi << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    mine = workloads.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)


def test_generators_are_seeded_and_chunk_stable():
    a = workloads.uniform_f32((300, 70000), 5)  # more than one draw chunk
    b = np.random.default_rng(5).uniform(-1, 1, size=(300, 70000)).astype(np.float32)
    assert np.array_equal(a, b)
    assert a.min() >= -1 and a.max() <= 1
    n = workloads.normal_bf16_bits((4, 5), 9)
    assert np.array_equal(n, workloads.normal_bf16_bits((4, 5), 9))
    v = oracle.bf16_bits_to_f64(workloads.normal_bf16_bits((512, 512), 1))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_generators_nd_shapes_and_conv_workloads():
    """N-D shapes draw the same values as their 2-D view (leading dimensions
    flattened), and every convolution workload draws tensors of its shapes."""
    a = workloads.uniform_f32((2, 3, 4, 5), 11)
    assert a.shape == (2, 3, 4, 5)
    assert np.array_equal(a.reshape(24, 5), workloads.uniform_f32((24, 5), 11))
    b = workloads.normal_bf16_bits((3, 2, 7), 12)
    assert b.shape == (3, 2, 7) and np.array_equal(b.reshape(6, 7), workloads.normal_bf16_bits((6, 7), 12))
    assert workloads.uniform_f32((9,), 1).shape == (9,)
    for c in workloads.CONV_WORKLOADS.values():
        if c.crs * c.p * c.q > 1 << 24:
            continue  # the full-size ones are drawn only where a GPU runs them
        assert c.x().shape == (c.batch, c.cin, c.h, c.w)
        assert c.weights().shape == (c.cout, c.cin, c.r, c.s)
        assert c.dy().shape == (c.batch, c.cout, c.p, c.q)


def test_nd_conv_workloads_match_the_oracle_shape():
    """Every N-D convolution workload: its output extents agree with the
    oracle's (the floor formula at stride and dilation 1), and the tensors it
    draws have the oracle's shapes."""
    from oracle.convnd import NdShape
    for c in workloads.CONVND_WORKLOADS.values():
        shape = NdShape(c.batch, c.cin, c.cout, c.size, c.kernel, c.pad, c.stride, c.dilation)
        assert shape.out == c.out == tuple(c.size), c.name  # "same" padding
        assert shape.crs == c.crs and shape.vol_out == c.vol_out
        assert c.x().shape == shape.x_shape
        assert c.weights().shape == shape.w_shape
        assert c.dy().shape == shape.y_shape
