"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (the default dispatch), at sampled positions: the plain product against
the oracle values stored in tests/golden/ (256 positions: corners, last row
and column, random), and the generalised-product variants against the oracle
computed one entry at a time.  The whole-output comparisons of the plain
product live in tests/test_whole_c.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from dense_gemm_03_amd import workloads as wl
from tests.golden.make_golden import read
from tests.gpu_util import TOL, log, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_full_size_sampled_against_golden(name):
    w = wl.WORKLOADS[name]
    log("[%s] drawing %dx%dx%d operands" % (name, w.M, w.N, w.K))
    A, B = w.operands()
    log("[%s] running on the GPU" % name)
    C = run(A, B).cpu().numpy()
    del A, B
    assert np.all(np.isfinite(C))
    _, _, I, J, C_ref, S = read(name)
    ratio = float(np.max(np.abs(C[I, J].astype(np.float64) - C_ref) / S))
    log("[%s] sampled max |C-C_ref|/S = %.3e (tol %.0e)" % (name, ratio, TOL[w.dtype]))
    assert ratio <= TOL[w.dtype]


# ------------------------------------------------- generalised-GEMM variants --

def _run_variant(w, A, B, C0):
    """w's product on the GPU (default dispatch): returns C as float64 and the
    raw output (float32 or bf16 bit patterns)."""
    import torch
    from tests.gpu_util import to_device
    import dense_gemm_03_amd as dg
    Ad, Bd = to_device(A), to_device(B)
    if C0 is not None:
        out = to_device(C0)
    else:
        out = torch.empty((w.M, w.N), device="cuda:0",
                          dtype=torch.float32 if w.out == "f32" else torch.bfloat16)
    dg.gemm(Ad, Bd, out=out, alpha=w.alpha, beta=w.beta, transa=w.transa, transb=w.transb)
    torch.cuda.synchronize()
    if w.out == "f32":
        raw = out.cpu().numpy()
        return raw.astype(np.float64), raw
    raw = out.cpu().view(torch.int16).numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(raw), raw


def _c0_f64(w, C0):
    if C0 is None:
        return None
    return C0.astype(np.float64) if w.out == "f32" else oracle.bf16_bits_to_f64(C0)


@pytest.mark.parametrize("name", list(wl.VARIANTS))
def test_variant_full_size_sampled(name):
    """Full-size generalised products (transposed operands, alpha/beta, bf16
    C) against the oracle at 256 sampled positions, within the tolerance
    (plus the bf16 output rounding for bf16 C)."""
    w = wl.VARIANTS[name]
    log("[%s] drawing operands %s %s" % (name, w.a_shape, w.b_shape))
    A, B = w.operands()
    C0 = w.initial_c() if w.beta != 0.0 else None
    C, _ = _run_variant(w, A, B, C0)
    assert np.all(np.isfinite(C))
    I, J = wl.sample_positions(w.M, w.N, 256, w.seed + 3000)
    c0 = _c0_f64(w, C0)
    kind = "f32" if w.dtype == "f32" else "bf16"
    C_ref, S = oracle.entries_general(A, B, I, J, w.alpha, w.beta,
                                      c0[I, J] if c0 is not None else None,
                                      w.transa, w.transb, kind=kind)
    bound = TOL[w.dtype] * S
    if w.out == "bf16":
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(C_ref)
    ratio = float(np.max(np.abs(C[I, J] - C_ref) / bound))
    log("[%s] sampled max err/bound = %.3e" % (name, ratio))
    assert ratio <= 1.0


@pytest.mark.parametrize("name", list(wl.VARIANTS))
def test_variant_full_size_exact_integers_sampled(name):
    """Integer operands and C of the variant's shapes: every intermediate is
    exact, so sampled entries equal the oracle bit for bit (bf16 C: the
    oracle's exact value rounded once to bf16)."""
    w = wl.VARIANTS[name]
    gen = wl.small_int_f32 if w.dtype == "f32" else wl.small_int_bf16_bits
    A, B = gen(w.a_shape, w.seed + 7), gen(w.b_shape, w.seed + 8)
    C0 = None
    if w.beta != 0.0:
        ints = np.random.default_rng(w.seed + 9).integers(-9, 10, size=(w.M, w.N))
        C0 = ints.astype(np.float32) if w.out == "f32" else \
            oracle.round_to_bf16_bits(ints.astype(np.float64))
    C, raw = _run_variant(w, A, B, C0)
    I, J = wl.sample_positions(w.M, w.N, 512, w.seed + 10)
    c0 = _c0_f64(w, C0)
    kind = "f32" if w.dtype == "f32" else "bf16"
    C_ref, _ = oracle.entries_general(A, B, I, J, w.alpha, w.beta,
                                      c0[I, J] if c0 is not None else None,
                                      w.transa, w.transb, kind=kind)
    if w.out == "bf16":
        want = oracle.round_to_bf16_bits(C_ref)
        got = raw[I, J]
    else:
        want, got = C_ref, C[I, J]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "%d sampled entries differ, first (%d,%d): %r vs %r" % (
        bad.size, I[bad[0]], J[bad[0]], got[bad[0]], want[bad[0]])
