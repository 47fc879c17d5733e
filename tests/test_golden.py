"""Golden sampled values: the seeded generators and the oracle reproduce them.

The files under tests/golden/ were written by make_golden.py from the oracle
alone; these CPU checks redraw the smaller workloads and recompute the sampled
entries, so a drifted random stream or a changed oracle sum shows up here.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_03_amd.workloads import WORKLOADS
from tests.golden.make_golden import digest, read


@pytest.mark.parametrize("name", ["fp32-256", "fp32-1000", "tall"])
def test_golden_reproduces(name):
    w = WORKLOADS[name]
    A, B = w.operands()
    shaA, shaB, I, J, C, S = read(name)
    assert digest(A) == shaA and digest(B) == shaB
    c, s = oracle.entries_f32(A, B, I, J)
    assert np.array_equal(c, C) and np.array_equal(s, S)


def test_golden_matches_full_product():
    w = WORKLOADS["fp32-256"]
    A, B = w.operands()
    _, _, I, J, C, S = read("fp32-256")
    Cf, Sf = oracle.gemm_f32(A, B)
    assert np.array_equal(Cf[I, J], C) and np.array_equal(Sf[I, J], S)


def test_every_workload_has_a_golden_file():
    for name in WORKLOADS:
        _, _, I, J, C, S = read(name)
        w = WORKLOADS[name]
        assert I.size == 256 and I.max() < w.M and J.max() < w.N and np.all(S > 0)
