"""Compile libjacobi.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m jacobi_stencil_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libjacobi.so")

SOURCES = ["libjacobi.hip", "kernels_sync.hip", "kernels_tblock.hip", "kernels_async.hip", "kernels_persist.hip",
           "kernels_probe.hip", "kernels_copy.hip"]

# -ffp-contract=off        : no fused multiply-add anywhere in the method's arithmetic
# -fno-fast-math           : no reassociation, no approximate division
# -fno-gpu-flush-denormals-to-zero : float32 subnormals are kept (they occur in the iterates)
# -fhip-fp32-correctly-rounded-divide-sqrt : '/' is the IEEE round-to-nearest quotient
# -packed-fp32-ops off     : no packed float32 instructions are generated
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def torch_lib_dir() -> str:
    """Directory of the HIP runtime bundled with PyTorch (found without importing torch)."""
    import importlib.util

    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("PyTorch is not installed; libjacobi shares its HIP runtime")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed ({proc.returncode}):\n{err}")
    if err and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object with hipcc, then link the shared library
    against the HIP runtime bundled with PyTorch (same soname as ROCm's), so the
    library uses only entry points that runtime has.  The Python binding loads
    torch first; the dynamic loader then binds libjacobi to that same runtime, so
    the process has one HIP runtime (one device context, shared streams)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    # the sources compile independently; a few at a time keeps the build to the longest one
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "6"))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        futs = [pool.submit(_run, [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
                for src, obj in zip(SOURCES, objs)]
        for f in futs:
            f.result()
    tlib = torch_lib_dir()
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, "-Wl,--no-undefined", "-L" + tlib, "-l:libamdhip64.so",
          "-lstdc++"], verbose)
    os.replace(tmp, LIB)
    return LIB


ABI_CLIENT_SRC = os.path.join(ROOT, "tests", "abi_client.c")
ABI_CLIENT = os.path.join(ROOT, "tests", "abi_client")


def build_abi_client(out: str = ABI_CLIENT, verbose: bool = False) -> str:
    """Compile tests/abi_client.c, a plain C11 caller of include/jacobi.h, with
    gcc against the built library and the HIP runtime the library uses (both
    found at run time through the rpath)."""
    tlib = torch_lib_dir()
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include", ABI_CLIENT_SRC, "-o", out,
          "-L" + HERE, "-l:libjacobi.so", "-L" + tlib, "-l:libamdhip64.so",
          "-Wl,-rpath," + HERE + ",-rpath," + tlib], verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
