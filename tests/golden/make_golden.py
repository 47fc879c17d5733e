"""Write the sampled full-size reference values under tests/golden/.

For every seeded workload (dense_gemm_03_amd.workloads.WORKLOADS) this draws the
operands, hashes them, and asks the oracle -- and nothing else -- for C_ref and
S at a fixed sample of output positions.  The files let the full-size GPU
parity tests check sampled outputs without re-running the oracle, and they pin
the input generators: a drifted random stream changes the operand hashes.

Run from the repository root:  python tests/golden/make_golden.py [name ...]
"""
from __future__ import annotations

import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from dense_gemm_03_amd.workloads import WORKLOADS, sample_positions  # noqa: E402

SAMPLES = 256
HERE = os.path.dirname(os.path.abspath(__file__))


def digest(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).view(np.uint8)).hexdigest()


def golden_path(name: str) -> str:
    return os.path.join(HERE, "sampled_%s.txt" % name)


def write(name: str) -> None:
    w = WORKLOADS[name]
    A, B = w.operands()
    I, J = sample_positions(w.M, w.N, SAMPLES, w.seed + 2000)
    fn = oracle.entries_f32 if w.dtype == "f32" else oracle.entries_bf16
    C, S = fn(A, B, I, J)
    with open(golden_path(name), "w") as f:
        f.write("# workload %s: %s M=%d N=%d K=%d dist=%s seed=%d (B seed %d)\n"
                % (name, w.dtype, w.M, w.N, w.K, w.dist, w.seed, w.seed + 1000))
        f.write("# written by tests/golden/make_golden.py from the oracle only\n")
        f.write("# sha256 A %s\n# sha256 B %s\n" % (digest(A), digest(B)))
        f.write("# columns: i j C_ref S  (C_ref and S as float.hex)\n")
        for t in range(I.size):
            f.write("%d %d %s %s\n" % (I[t], J[t], float(C[t]).hex(), float(S[t]).hex()))


def read(name: str):
    """(sha_A, sha_B, I, J, C_ref, S) from a golden file."""
    sha = {}
    rows = []
    with open(golden_path(name)) as f:
        for line in f:
            if line.startswith("# sha256 "):
                _, _, which, h = line.split()
                sha[which] = h
            elif not line.startswith("#"):
                i, j, c, s = line.split()
                rows.append((int(i), int(j), float.fromhex(c), float.fromhex(s)))
    I = np.array([r[0] for r in rows], dtype=np.int64)
    J = np.array([r[1] for r in rows], dtype=np.int64)
    C = np.array([r[2] for r in rows])
    S = np.array([r[3] for r in rows])
    return sha["A"], sha["B"], I, J, C, S


if __name__ == "__main__":
    names = sys.argv[1:] or list(WORKLOADS)
    for n in names:
        write(n)
        print("wrote", golden_path(n))
