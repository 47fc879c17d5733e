"""Helpers shared by the GPU tests: move seeded numpy operands to the device,
run the library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import dense_gemm_03_amd as dg
import oracle

TOL = {"f32": 1e-5, "bf16": 4e-3}
# Far inside the tolerance; larger ratios are printed as a diagnostic (random
# fp32-accumulated sums land near 1e-7), not failed.
DIAGNOSTIC = 1e-6


def log(*args):
    print(*args, flush=True)
    sys.stdout.flush()


# Lines printed in the terminal summary at the end of the run (after the
# captured output of passing tests is gone): the headline parity results.
SUMMARY: list[str] = []


def report(line: str):
    """log() now, and repeat the line in the run's terminal summary."""
    log(line)
    SUMMARY.append(line)


def to_device(x: np.ndarray):
    """float32 -> torch.float32 and uint16 bf16 patterns -> torch.bfloat16 on cuda:0."""
    import torch
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    raise TypeError(x.dtype)


def run(A: np.ndarray, B: np.ndarray, cfg=None, split_k=0, out=None, pad_a=0, pad_b=0, fill=None):
    """C = A . B on the GPU through the C ABI; returns the torch output (synchronised).

    pad_a / pad_b > 0 store the operand on the device with that many extra
    columns per row (leading dimension cols + pad), filled with ``fill``."""
    import torch
    Ad, Bd = to_device(_padded(A, pad_a, fill)), to_device(_padded(B, pad_b, fill))
    Ad, Bd = Ad[:, :A.shape[1]], Bd[:, :B.shape[1]]
    C = dg.gemm(Ad, Bd, out=out, cfg=cfg, split_k=split_k)
    torch.cuda.synchronize()
    return C


def _padded(x: np.ndarray, extra: int, fill):
    if extra == 0:
        return x
    buf = np.full((x.shape[0], x.shape[1] + extra), fill, dtype=x.dtype)
    buf[:, :x.shape[1]] = x
    return buf


def reference(A: np.ndarray, B: np.ndarray):
    return oracle.gemm_f32(A, B) if A.dtype == np.float32 else oracle.gemm_bf16(A, B)


def check_close(C_gpu: np.ndarray, A: np.ndarray, B: np.ndarray, what: str):
    """Assert max |C - C_ref| / S within the dtype's tolerance (and exact zeros
    where S == 0); print the ratio."""
    dt = "f32" if A.dtype == np.float32 else "bf16"
    C_ref, S = reference(A, B)
    ratio, zeros_ok = oracle.max_error_ratio(C_gpu, C_ref, S)
    log("  %s: max |C-C_ref|/S = %.3e (tol %.0e)%s" % (
        what, ratio, TOL[dt], "  [diagnostic: above %.0e]" % DIAGNOSTIC if ratio > DIAGNOSTIC else ""))
    assert zeros_ok, "%s: nonzero output where every product is zero" % what
    assert ratio <= TOL[dt], "%s: error ratio %.3e above %.0e" % (what, ratio, TOL[dt])
    return ratio


def check_exact(C_gpu: np.ndarray, A: np.ndarray, B: np.ndarray, what: str):
    """Integer-valued operands: every partial sum is exact, so the GPU result
    must equal the oracle bit for bit."""
    C_ref, _ = reference(A, B)
    bad = np.argwhere(C_gpu.astype(np.float64) != C_ref)
    assert bad.size == 0, "%s: %d entries differ, first at %s: gpu %r oracle %r" % (
        what, len(bad), tuple(bad[0]), C_gpu[tuple(bad[0])], C_ref[tuple(bad[0])])
