"""Build the HIP library ``libdense_gemm.so`` for gfx950 with hipcc, in-tree.

Usage:  python -m dense_gemm_03_amd.build   (or dense_gemm_03_amd.build.build())

Every source compiles to its own object in parallel, then one shared library
is linked next to this file.  The build always recompiles: it is the "does it
build" check as well as the build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdense_gemm.so")

# (source, object name, extra defines).  gemm_instances.hip is compiled once
# per input type and operand layout, so the kernel instantiations build in
# parallel.
SOURCES = [("gemm_api.hip", "gemm_api", []),
           ("gemm_tables.hip", "gemm_tables", []),
           ("gemm_aux.hip", "gemm_aux", []),
           ("conv.hip", "conv", [])]
for _dtype in ("F32", "BF16"):
    for _layout in ("NN", "NT", "TN", "TT", "CF", "CW", "CFT", "CWT", "C3F", "C3W", "CFP", "CWP",
                    "C3FP", "C3WP", "CFW", "CWW", "C4F", "C4W", "C4FP", "C4WP"):
        SOURCES.append(("gemm_instances.hip", "gemm_%s_%s" % (_dtype.lower(), _layout.lower()),
                        ["DG_DTYPE_TABLE=DG_%s_TABLE" % _dtype, "DG_LAYOUT=" + _layout]))

ARCH = "gfx950"
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Werror",
    # No packed-fp32 instructions anywhere in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the GEMM library")
    return path


def _compile(item) -> str:
    src, name, defines = item
    obj = os.path.join(OBJDIR, name + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *["-D" + d for d in defines], "-I", INCLUDE, "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that
    # note is expected.  Anything else is printed.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s (%s):\n%s" % (src, name, "\n".join(msgs)))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
