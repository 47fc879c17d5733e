"""The generalised-GEMM oracle and the bf16 output rounding against their pins
(CPU only).

``oracle.gemm_general`` computes alpha * op(A) . op(B) + beta * C0 ("Learning
to develop for GPUs through the GEMM operation", section "Generalized matrix
multiplication GEMM").  Its pins do not retype that formula: they are a
reduction to the already-pinned plain product, closed forms (rank-one operands
whose product factorises, all-ones operands), the transpose identity
(op(A) op(B))^T = op(B)^T op(A)^T, and the conventions for alpha == 0 and
beta == 0 shown through NaN operands that must not be read.  Mutants with
planted mistakes must each fail at least one pin.

``oracle.round_to_bf16_bits`` is pinned by hand-derived roundings (ties to
even, subnormals, overflow, NaN) and by agreement with torch's float32 ->
bfloat16 conversion on random values.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle


class PinFailure(AssertionError):
    pass


def _check(cond, msg):
    if not cond:
        raise PinFailure(msg)


TRANS = list(itertools.product([False, True], [False, True]))


def _stored(op_matrix: np.ndarray, trans: bool) -> np.ndarray:
    """The stored matrix whose op() is `op_matrix`."""
    return np.ascontiguousarray(op_matrix.T if trans else op_matrix, dtype=np.float32)


# ------------------------------------------------------------------- pins --

def pin_reduces_to_product(general):
    """alpha = 1, beta = 0, no transposes: the plain product, C and S bit for bit."""
    rng = np.random.default_rng(3)
    A = rng.uniform(-1, 1, size=(7, 9)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(9, 5)).astype(np.float32)
    C, S = general(A, B, 1.0, 0.0, None, False, False)
    Cp, Sp = oracle.gemm_f32(A, B, threads=2)
    _check(np.array_equal(C, Cp) and np.array_equal(S, Sp), "plain case differs from the product")


def pin_rank_one_closed_form(general):
    """op(A)[i][k] = a_i p_k and op(B)[k][j] = q_k b_j give
    C[i][j] = alpha * a_i b_j (p . q) + beta * C0[i][j] and
    S[i][j] = |alpha| |a_i| |b_j| (|p| . |q|) + |beta| |C0[i][j]|, for every
    transpose combination, on rectangular and square shapes."""
    rng = np.random.default_rng(5)
    for (M, N, K) in [(3, 4, 5), (4, 4, 4), (6, 2, 3)]:
        a = rng.integers(-4, 5, size=M).astype(np.float64)
        b = rng.integers(-4, 5, size=N).astype(np.float64)
        p = rng.integers(-3, 4, size=K).astype(np.float64)
        q = rng.integers(-3, 4, size=K).astype(np.float64)
        # make the factors distinguishable from their transposes / reversals
        a[0], b[-1], p[0], q[-1] = 7.0, -5.0, 2.0, 3.0
        C0 = rng.integers(-9, 10, size=(M, N)).astype(np.float64)
        opA, opB = np.outer(a, p), np.outer(q, b)
        for ta, tb in TRANS:
            for alpha, beta in [(3.0, -2.0), (-0.5, 0.25), (1.0, 0.0)]:
                C, S = general(_stored(opA, ta), _stored(opB, tb), alpha, beta,
                               C0 if beta != 0.0 else None, ta, tb)
                C_exp = alpha * np.outer(a, b) * float(p @ q) + beta * C0
                S_exp = abs(alpha) * np.outer(np.abs(a), np.abs(b)) * float(np.abs(p) @ np.abs(q)) \
                    + abs(beta) * np.abs(C0)
                _check(C.shape == (M, N), "shape %s for %s" % (C.shape, (M, N)))
                _check(np.array_equal(C, C_exp), "rank-one C wrong (ta=%s tb=%s)" % (ta, tb))
                _check(np.array_equal(S, S_exp), "rank-one S wrong (ta=%s tb=%s)" % (ta, tb))


def pin_all_ones(general):
    """All-ones operands and C0: C = alpha * K + beta everywhere."""
    for (M, N, K) in [(2, 3, 7), (5, 1, 4)]:
        for ta, tb in TRANS:
            A = np.ones((K, M) if ta else (M, K), dtype=np.float32)
            B = np.ones((N, K) if tb else (K, N), dtype=np.float32)
            C, _ = general(A, B, 2.0, 3.0, np.ones((M, N)), ta, tb)
            _check(C.shape == (M, N) and np.all(C == 2.0 * K + 3.0), "all-ones case wrong")


def pin_alpha_zero_reads_nothing(general):
    """alpha == 0: C = beta * C0 and A, B (all NaN here) are not read."""
    A = np.full((4, 3), np.nan, dtype=np.float32)
    B = np.full((3, 2), np.nan, dtype=np.float32)
    C0 = np.array([[1.0, -2.0], [3.0, 4.0], [-5.0, 6.0], [7.0, 0.0]])
    C, S = general(A, B, 0.0, 0.5, C0, False, False)
    _check(np.array_equal(C, 0.5 * C0) and np.array_equal(S, 0.5 * np.abs(C0)),
           "alpha == 0 must give beta * C0")


def pin_beta_zero_ignores_c0(general):
    """beta == 0: C0 (all NaN here) is not read."""
    A = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    B = np.array([[1.0, 0.0], [0.0, 1.0]], dtype=np.float32)
    C, S = general(A, B, 2.0, 0.0, np.full((2, 2), np.nan), False, False)
    _check(np.array_equal(C, 2.0 * A.astype(np.float64)), "beta == 0 must not read C0")
    _check(np.all(np.isfinite(S)), "beta == 0 must not put C0 into S")


def pin_transpose_identity(general):
    """(op(A) op(B))^T = op(B)^T op(A)^T with the same k order: bit for bit,
    on random values (so a mixed-up operand or flag changes the result)."""
    rng = np.random.default_rng(9)
    M, N, K = 5, 4, 6
    for ta, tb in TRANS:
        A = rng.uniform(-1, 1, size=(K, M) if ta else (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(N, K) if tb else (K, N)).astype(np.float32)
        C0 = rng.uniform(-1, 1, size=(M, N))
        C, S = general(A, B, 1.5, -0.75, C0, ta, tb)
        # op(B)^T is B with the opposite flag, op(A)^T likewise
        Ct, St = general(B, A, 1.5, -0.75, np.ascontiguousarray(C0.T), not tb, not ta)
        _check(np.array_equal(C, Ct.T) and np.array_equal(S, St.T), "transpose identity fails")


ALL_PINS = [pin_reduces_to_product, pin_rank_one_closed_form, pin_all_ones,
            pin_alpha_zero_reads_nothing, pin_beta_zero_ignores_c0, pin_transpose_identity]


def _real(A, B, alpha, beta, C0, ta, tb):
    return oracle.gemm_general(A, B, alpha, beta, C0, ta, tb, kind="f32", threads=2)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_real)


# ---------------------------------------------------------------- mutants --

def _mutant(name):
    def transa_ignored_if_square(A, B, alpha, beta, C0, ta, tb):
        return _real(A, B, alpha, beta, C0, ta and A.shape[0] != A.shape[1], tb)

    def transb_flipped_if_square(A, B, alpha, beta, C0, ta, tb):
        return _real(A, B, alpha, beta, C0, ta, (not tb) if B.shape[0] == B.shape[1] else tb)

    def alpha_beta_swapped(A, B, alpha, beta, C0, ta, tb):
        if C0 is None or alpha == 0.0:
            return _real(A, B, alpha, beta, C0, ta, tb)
        P, SP = _real(A, B, 1.0, 0.0, None, ta, tb)
        return beta * P + alpha * np.asarray(C0), SP

    def c0_read_when_beta_zero(A, B, alpha, beta, C0, ta, tb):
        C, S = _real(A, B, alpha, beta, C0, ta, tb)
        if beta == 0.0 and C0 is not None:
            C = C + beta * np.asarray(C0)
        return C, S

    def beta_term_dropped(A, B, alpha, beta, C0, ta, tb):
        return _real(A, B, alpha, 0.0, None, ta, tb)

    def s_without_alpha(A, B, alpha, beta, C0, ta, tb):
        C, _ = _real(A, B, alpha, beta, C0, ta, tb)
        _, SP = _real(A, B, 1.0, 0.0, None, ta, tb) if alpha != 0.0 else (None, np.zeros_like(C))
        return C, SP + (abs(beta) * np.abs(np.asarray(C0)) if beta != 0.0 else 0.0)

    def product_read_when_alpha_zero(A, B, alpha, beta, C0, ta, tb):
        C, S = _real(A, B, alpha, beta, C0, ta, tb)
        if alpha == 0.0:
            P, _ = _real(A, B, 1.0, 0.0, None, ta, tb)
            C = C + alpha * P
        return C, S

    return locals()[name]


MUTANTS = ["transa_ignored_if_square", "transb_flipped_if_square", "alpha_beta_swapped",
           "c0_read_when_beta_zero", "beta_term_dropped", "s_without_alpha",
           "product_read_when_alpha_zero"]


@pytest.mark.parametrize("name", MUTANTS)
def test_pins_catch_planted_mistake(name):
    mutant = _mutant(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (PinFailure, ValueError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name


def test_bf16_kind_matches_f32_kind_on_bf16_values():
    """The bf16 encoding of the same (bf16-representable) values gives the
    same result as the fp32 encoding, for every transpose combination."""
    rng = np.random.default_rng(11)
    for ta, tb in TRANS:
        A = rng.integers(-8, 9, size=(6, 4) if ta else (4, 6)).astype(np.float32) / 4
        B = rng.integers(-8, 9, size=(5, 6) if tb else (6, 5)).astype(np.float32) / 8
        C0 = rng.integers(-8, 9, size=(4, 5)).astype(np.float64)
        Af = oracle.gemm_general(A, B, 1.25, -3.0, C0, ta, tb, kind="f32")
        bits = lambda X: (X.view(np.uint32) >> 16).astype(np.uint16)
        Ab = oracle.gemm_general(bits(A), bits(B), 1.25, -3.0, C0, ta, tb, kind="bf16")
        assert np.array_equal(Af[0], Ab[0]) and np.array_equal(Af[1], Ab[1])


def test_k_zero_and_shape_errors():
    C, S = oracle.gemm_general(np.zeros((3, 0), np.float32), np.zeros((0, 2), np.float32),
                               2.0, 0.5, np.full((3, 2), 4.0))
    assert np.array_equal(C, np.full((3, 2), 2.0)) and np.array_equal(S, np.full((3, 2), 2.0))
    with pytest.raises(ValueError):
        oracle.gemm_general(np.zeros((3, 4), np.float32), np.zeros((3, 2), np.float32))
    with pytest.raises(ValueError):
        oracle.gemm_general(np.zeros((3, 4), np.float32), np.zeros((4, 2), np.float32), beta=1.0)


# ------------------------------------------------------------ bf16 rounding --

def test_round_to_bf16_hand_values():
    """Roundings derived by hand: bf16 keeps 8 significant bits.
    257 = 256 + 1 lies halfway between 256 and 258 -> the even significand, 256;
    259 halfway between 258 and 260 -> 260 (even); 1 + 2^-8 halfway between 1
    and 1 + 2^-7 -> 1; 1 + 3*2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 ->
    1 + 2^-6; 1 + 2^-8 + 2^-20 above the midpoint -> 1 + 2^-7; 2^-130 is the
    subnormal 8 * 2^-133; the largest bf16 (2 - 2^-7) 2^127 stays; halfway
    above it rounds to infinity; NaN stays NaN; signs are kept."""
    cases = [
        (257.0, 0x4380), (259.0, 0x4382), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81), (2.0 ** -130, 0x0008), (-1.5, 0xBFC0),
        ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F), ((2.0 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),
        (-0.0, 0x8000), (0.0, 0x0000), (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
    ]
    got = oracle.round_to_bf16_bits(np.array([x for x, _ in cases]))
    for (x, want), g in zip(cases, got):
        assert int(g) == want, "round(%r) = %#06x, want %#06x" % (x, int(g), want)
    assert (int(oracle.round_to_bf16_bits(np.nan)) & 0x7FFF) > 0x7F80


def test_round_to_bf16_matches_torch_on_float32():
    """On float32 inputs the rounding agrees with torch's bfloat16 conversion
    (round to nearest even), including values at exact midpoints."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    mid = ((rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, mid[np.isfinite(mid)]])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_to_bf16_matches_exact_rational_rounding():
    """float64 values that binary32 cannot hold (so torch's conversion, which
    starts from binary32, does not apply): the bf16 pattern equals rounding
    the exact value with Python fractions -- the multiple of 2^(e-8) (at
    least 2^-133) nearest to it, ties to even -- packed through binary32."""
    import math
    import struct
    from fractions import Fraction
    rng = np.random.default_rng(31)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-95, 95, 3000))
    x = np.concatenate([x, (rng.integers(-(1 << 20), 1 << 20, 500) + 0.5) * 2.0 ** -12,
                        [2.0 ** -140, -3 * 2.0 ** -135, 3.4e38, -3.5e38]])
    got = oracle.round_to_bf16_bits(x)
    for v, g in zip(x, got):
        m, e = math.frexp(abs(v))
        sp = max(e - 8, -133)
        q = round(Fraction(abs(v)) / Fraction(2) ** sp)       # round half to even
        val = Fraction(q) * Fraction(2) ** sp
        if val >= Fraction(2) ** 128:
            want = 0x7F80
        else:
            want = struct.unpack(">I", struct.pack(">f", float(val)))[0] >> 16
        if v < 0:
            want |= 0x8000
        assert int(g) == want, "round(%r) = %#06x, want %#06x" % (v, int(g), want)


def test_entries_general_match_full_product_bitwise():
    """The one-entry-at-a-time form equals the full generalised product at
    the same positions, bit for bit (same k order), for every transpose
    combination and both encodings."""
    rng = np.random.default_rng(21)
    M, N, K = 37, 29, 53
    I = rng.integers(0, M, 60)
    J = rng.integers(0, N, 60)
    for ta, tb in TRANS:
        A = rng.uniform(-1, 1, size=(K, M) if ta else (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(N, K) if tb else (K, N)).astype(np.float32)
        C0 = rng.uniform(-1, 1, size=(M, N))
        for kind in ("f32", "bf16"):
            a, b = (A, B) if kind == "f32" else (
                (A.view(np.uint32) >> 16).astype(np.uint16), (B.view(np.uint32) >> 16).astype(np.uint16))
            for alpha, beta in [(0.75, -1.5), (1.0, 0.0), (0.0, 2.0)]:
                C, S = oracle.gemm_general(a, b, alpha, beta, C0, ta, tb, kind=kind)
                Ce, Se = oracle.entries_general(a, b, I, J, alpha, beta, C0[I, J], ta, tb, kind=kind)
                assert np.array_equal(C[I, J], Ce) and np.array_equal(S[I, J], Se)
