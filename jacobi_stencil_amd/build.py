"""Compile libjacobi.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m jacobi_stencil_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libjacobi.so")

SOURCES = ["libjacobi.hip", "kernels_sync.hip"]

# -ffp-contract=off        : no fused multiply-add anywhere in the method's arithmetic
# -fno-fast-math           : no reassociation, no approximate division
# -fno-gpu-flush-denormals-to-zero : float32 subnormals are kept (they occur in the iterates)
# -fhip-fp32-correctly-rounded-divide-sqrt : '/' is the IEEE round-to-nearest quotient
# -packed-fp32-ops off     : no packed float32 instructions are generated
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
