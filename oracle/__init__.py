"""Plain CPU reference ("the oracle") for the backward-Euler five-point Jacobi solve.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The library path
(``jacobi_stencil_amd``) never imports, links or runs anything here, and this
package imports nothing from it.

The arithmetic lives in ``jacobi_oracle.c`` (serial C with OpenMP over rows,
float32, no contraction); this module only builds it and marshals numpy arrays.
What each function computes follows the page "stencil-jacobian.vercel.app",
sections 01 ("The problem") and 02 ("Method"); see the header comment of
``jacobi_oracle.c`` for the exact operation order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jacobi_oracle.c")
_LIB = os.path.join(_HERE, "libjacobi_oracle.so")

SYNC = 0
ASYNC = 2
# negative control: b re-formed from the current iterate before every sweep
WRONG_B = 3
# depth controllers for ASYNC (page "stencil-jacobian.vercel.app", section 02)
STATIC, G_ASC, G_DESC, SCHED = 0, 1, 2, 3
OK, EINVAL, ENOMEM, ENOCONV, ENAN = 0, -1, -2, -4, -5

# -ffp-contract=off: GCC fuses a*b+c by default for GNU dialects; the pages fix
# separate round-to-nearest operations.  No -ffast-math: it would enable
# reassociation and flush subnormals to zero.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-fPIC", "-shared"]


def build() -> str:
    """Compile the oracle into ``oracle/libjacobi_oracle.so`` (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        # JACOBI_ORACLE_LIB points the tests at a deliberately broken copy of
        # the oracle (tests/test_oracle_mutants.py); unset, the real one loads.
        path = os.environ.get("JACOBI_ORACLE_LIB", _LIB)
        if path == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_get_threads.restype = ctypes.c_int
        lib.orc_diag.argtypes = [ctypes.c_float]
        lib.orc_diag.restype = ctypes.c_float
        lib.orc_rhs.argtypes = [ctypes.c_int, f32p, f32p, f32p]
        lib.orc_rhs_norm.argtypes = [ctypes.c_int, ctypes.c_float, f32p]
        lib.orc_rhs_norm.restype = ctypes.c_float
        lib.orc_sweep.argtypes = [ctypes.c_int, ctypes.c_float, f32p, f32p, f32p]
        lib.orc_residual.argtypes = [ctypes.c_int, ctypes.c_float, f32p, f32p]
        lib.orc_residual.restype = ctypes.c_float
        lib.orc_async_launch.argtypes = [ctypes.c_int, ctypes.c_float, f32p, f32p, f32p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.orc_solve.argtypes = [ctypes.c_int, ctypes.c_float, f32p, f32p, ctypes.c_int,
                                  ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int64, i64p, f32p,
                                  ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_int64)]
        lib.orc_solve.restype = ctypes.c_int
        lib.orc_solve_ex.argtypes = [ctypes.c_int, ctypes.c_float, f32p, f32p, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int64, i64p, f32p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.POINTER(ctypes.c_int64)]
        lib.orc_solve_ex.restype = ctypes.c_int
        _lib = lib
    return _lib


def _grid(a, N):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.shape != (N, N):
        raise ValueError(f"expected an {N}x{N} array, got {a.shape}")
    return a


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


def diag(r: float) -> np.float32:
    """d = 1 + 4r in two float32 operations."""
    return np.float32(_load().orc_diag(np.float32(r)))


def rhs(u, s):
    """b = u^n + s (s = dt*f), one float32 add per point."""
    N = np.asarray(u).shape[0]
    b = np.empty((N, N), np.float32)
    _load().orc_rhs(N, _grid(u, N), _grid(s, N), b)
    return b


def rhs_norm(b, r) -> np.float32:
    """bA = max |b + r*g|, g = 100 on the row next to the top boundary."""
    N = np.asarray(b).shape[0]
    return np.float32(_load().orc_rhs_norm(N, np.float32(r), _grid(b, N)))


def sweep(u, b, r):
    """One point-Jacobi sweep u' = (b + r*(((uE+uW)+uN)+uS)) / (1+4r)."""
    N = np.asarray(u).shape[0]
    out = np.empty((N, N), np.float32)
    _load().orc_sweep(N, np.float32(r), _grid(u, N), _grid(b, N), out)
    return out


def residual(u, b, r) -> np.float32:
    """R = max |(b - C) + r*(((E-C)+(W-C))+(N-C))+(S-C))|; NaN if any term is NaN."""
    N = np.asarray(u).shape[0]
    return np.float32(_load().orc_residual(N, np.float32(r), _grid(u, N), _grid(b, N)))


def async_launch(u, b, r, tx, ty, D, o=0):
    """One block-asynchronous launch: tiles tx x ty, each worked on widened by o
    overlap cells per side, frozen one-cell halo around that, D sweeps; each
    tile writes back only its own points."""
    N = np.asarray(u).shape[0]
    out = np.empty((N, N), np.float32)
    _load().orc_async_launch(N, np.float32(r), _grid(u, N), _grid(b, N), out, int(tx), int(ty), int(D), int(o))
    return out


class Result:
    """Outcome of ``solve``: final field, per-step sweeps and rho, every check's R."""

    def __init__(self, u, sweeps, rho, status, R_log, D_log=None):
        self.u = u
        self.sweeps = sweeps
        self.rho = rho
        self.status = status
        self.R_log = R_log
        self.D_log = D_log  # depth of every check interval (solve with log_cap > 0)

    @property
    def total_sweeps(self) -> int:
        return int(self.sweeps.sum())


def solve(N, r, s, u0=None, steps=10, tol=1e-5, M=8, mode=SYNC, D=1, tx=32, ty=8,
          max_sweeps=10**6, log_cap=0, o=0, controller=STATIC, schedule=None) -> Result:
    """``steps`` backward-Euler steps, each Jacobi-iterated until rho < tol (checked every M).

    ASYNC options: tiles tx x ty widened by ``o`` overlap cells; ``controller``
    picks each interval's depth (STATIC: D; G_ASC / G_DESC: from the previous
    check's rho, at most D; SCHED: ``schedule[i]`` for the i-th interval)."""
    lib = _load()
    s = _grid(s, N)
    u = np.zeros((N, N), np.float32) if u0 is None else _grid(u0, N).copy()
    sweeps = np.zeros(max(steps, 1), np.int64)
    rho = np.zeros(max(steps, 1), np.float32)
    log = np.zeros(max(log_cap, 1), np.float32)
    dlog = np.zeros(max(log_cap, 1), np.int32)
    nlog = ctypes.c_int64(0)
    sched = None
    nsched = 0
    if schedule is not None:
        sched = np.ascontiguousarray(schedule, dtype=np.int32)
        nsched = len(sched)
    status = lib.orc_solve_ex(int(N), np.float32(r), s, u, int(steps), np.float32(tol), int(M),
                              int(mode), int(D), int(tx), int(ty), int(o), int(controller),
                              sched.ctypes.data if sched is not None else None, int(nsched),
                              int(max_sweeps), sweeps, rho,
                              log.ctypes.data if log_cap > 0 else None,
                              dlog.ctypes.data if log_cap > 0 else None, int(log_cap),
                              ctypes.byref(nlog))
    n = min(int(nlog.value), log_cap)
    return Result(u, sweeps[:steps], rho[:steps], int(status), log[:n].copy(), dlog[:n].copy())
