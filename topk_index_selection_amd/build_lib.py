"""Build ``libltopk.so`` in-tree with hipcc for gfx950.

    python -m topk_index_selection_amd.build_lib

The library is two HIP translation units (the selection kernels with their C
ABI, and the output variants with theirs). All HIP code is built with
packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ltopk_kernels.hip")
SOURCES = [SRC, os.path.join(PKG, "csrc", "ltopk_output.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libltopk.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The streaming kernel's ring of sweeps in flight lives in registers only
    # if its loop is fully unrolled; with a compaction inlined at every stage
    # the body exceeds the default size limit for a requested full unroll.
    "-mllvm", "-pragma-unroll-threshold=65536",
]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles). Returns the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I" + INC, "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, out))
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
