"""Python binding of libjacobi (include/jacobi.h): argument marshalling only.

Every step of the solve runs in the HIP kernels of ``libjacobi.so``; this
module converts arguments, nothing more.  If the library has not been built
(``python -m jacobi_stencil_amd.build``) every call raises: there is no other
implementation to fall back to.

The functions keep the C names and return the C status code first.  ``Solver``
is a convenience wrapper that takes its workspace and stream from PyTorch
(device memory and stream plumbing only) and raises ``JacobiError`` on failure.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjacobi.so")

JAC_OK, JAC_EINVAL, JAC_ENOMEM, JAC_EDEVICE, JAC_ENOCONV, JAC_ENAN = 0, -1, -2, -3, -4, -5
JAC_SYNC, JAC_TBLOCK, JAC_ASYNC, JAC_SYNC_UNFUSED = 0, 1, 2, 3
JAC_LAUNCH, JAC_GRAPH, JAC_PERSISTENT = 0, 1, 2
JAC_CHECKS_OVERLAPPED, JAC_CHECKS_BLOCKING = 0, 1
JAC_STATIC, JAC_G_ASC, JAC_G_DESC, JAC_G_FB = 0, 1, 2, 3
KCLASS = {"rhs": 0, "sync": 1, "sync_check": 2, "tblock": 3, "async": 4, "residual": 5, "persistent": 6,
          "noop": 7, "reduce": 8, "tblock_rhs": 9, "tblock_part": 10}
STATUS_NAMES = {0: "JAC_OK", -1: "JAC_EINVAL", -2: "JAC_ENOMEM", -3: "JAC_EDEVICE", -4: "JAC_ENOCONV",
                -5: "JAC_ENAN"}

EXPORTS = ("jac_opts_default", "jac_workspace_bytes", "jac_create", "jac_step", "jac_solve", "jac_sweep",
           "jac_sweep_static",
           "jac_get_field", "jac_set_field", "jac_reset", "jac_fast_division", "jac_last_division", "jac_depth_log",
           "jac_destroy", "jac_last_error",
           "jac_profile", "jac_profile_read", "jac_stream_probe")


class jac_opts(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("driver", ctypes.c_int32), ("D", ctypes.c_int32),
                ("tile_x", ctypes.c_int32), ("tile_y", ctypes.c_int32), ("M", ctypes.c_int32),
                ("tol", ctypes.c_float), ("band_rows", ctypes.c_int32), ("max_sweeps", ctypes.c_int64),
                ("checks", ctypes.c_int32), ("controller", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class JacobiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library():
    """Load libjacobi.so from the package directory; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m jacobi_stencil_amd.build`")
        # torch's HIP runtime must be loaded first: libjacobi's dependency on
        # libamdhip64.so.7 then binds to it, and the process has one runtime
        # whose streams and memory both sides share.
        import torch  # noqa: F401

        lib = ctypes.CDLL(LIB_PATH)
        vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
        lib.jac_opts_default.argtypes = [ctypes.POINTER(jac_opts)]
        lib.jac_opts_default.restype = None
        lib.jac_workspace_bytes.argtypes = [ctypes.c_int]
        lib.jac_workspace_bytes.restype = ctypes.c_size_t
        lib.jac_create.argtypes = [ctypes.c_int, f32, vp, vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
        lib.jac_step.argtypes = [vp, ctypes.POINTER(jac_opts), ctypes.POINTER(i64), ctypes.POINTER(f32)]
        lib.jac_solve.argtypes = [vp, ctypes.c_int, ctypes.POINTER(jac_opts), vp, vp]
        lib.jac_sweep.argtypes = [vp, ctypes.POINTER(jac_opts), i64, ctypes.POINTER(f32)]
        lib.jac_sweep_static.argtypes = [vp, ctypes.POINTER(jac_opts), i64, ctypes.POINTER(f32)]
        lib.jac_get_field.argtypes = [vp, vp]
        lib.jac_set_field.argtypes = [vp, vp]
        lib.jac_reset.argtypes = [vp]
        lib.jac_fast_division.argtypes = [vp]
        lib.jac_last_division.argtypes = [vp]
        lib.jac_depth_log.argtypes = [vp, vp, i64, ctypes.POINTER(i64)]
        lib.jac_stream_probe.argtypes = [vp, vp, vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        lib.jac_destroy.argtypes = [vp]
        lib.jac_last_error.argtypes = []
        lib.jac_last_error.restype = ctypes.c_char_p
        lib.jac_profile.argtypes = [vp, ctypes.c_int]
        lib.jac_profile_read.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(i64), ctypes.POINTER(i64)]
        for name in EXPORTS:
            if name not in ("jac_opts_default", "jac_workspace_bytes", "jac_last_error"):
                getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


# ------------------------------------------------------------------ C names

def jac_opts_default(**overrides) -> jac_opts:
    o = jac_opts()
    load_library().jac_opts_default(ctypes.byref(o))
    for k, v in overrides.items():
        setattr(o, k, v)
    return o


def jac_workspace_bytes(N: int) -> int:
    return int(load_library().jac_workspace_bytes(int(N)))


def jac_last_error() -> str:
    return load_library().jac_last_error().decode()


def jac_create(N: int, r: float, source_host, workspace_ptr: int, ws_bytes: int, stream_ptr: int):
    """Returns (status, ctx).  source_host: N x N float32 array or None."""
    src = None
    if source_host is not None:
        src = np.ascontiguousarray(source_host, dtype=np.float32)
        if src.shape != (N, N):
            raise ValueError(f"source must be {N}x{N}")
    h = ctypes.c_void_p()
    st = load_library().jac_create(int(N), ctypes.c_float(r), src.ctypes.data if src is not None else None,
                                   ctypes.c_void_p(workspace_ptr), int(ws_bytes), ctypes.c_void_p(stream_ptr),
                                   ctypes.byref(h))
    return st, h


def jac_step(ctx, opts: jac_opts):
    """Returns (status, sweeps, rho)."""
    k = ctypes.c_int64(0)
    rho = ctypes.c_float(0)
    st = load_library().jac_step(ctx, ctypes.byref(opts), ctypes.byref(k), ctypes.byref(rho))
    return st, int(k.value), float(rho.value)


def jac_solve(ctx, nsteps: int, opts: jac_opts):
    """Returns (status, sweeps[nsteps] int64, rho[nsteps] float32)."""
    sweeps = np.zeros(max(nsteps, 1), np.int64)
    rho = np.zeros(max(nsteps, 1), np.float32)
    st = load_library().jac_solve(ctx, int(nsteps), ctypes.byref(opts), sweeps.ctypes.data, rho.ctypes.data)
    return st, sweeps[:nsteps], rho[:nsteps]


def jac_sweep(ctx, opts: jac_opts, nsweeps: int, want_rho: bool = False):
    """Returns (status, rho or None)."""
    rho = ctypes.c_float(0)
    st = load_library().jac_sweep(ctx, ctypes.byref(opts), int(nsweeps), ctypes.byref(rho) if want_rho else None)
    return st, (float(rho.value) if want_rho else None)


def jac_sweep_static(ctx, opts: jac_opts, nsweeps: int, want_rho: bool = False):
    """jac_sweep with the library's static device scratch (allocates nothing).
    Returns (status, rho or None)."""
    rho = ctypes.c_float(0)
    st = load_library().jac_sweep_static(ctx, ctypes.byref(opts), int(nsweeps),
                                         ctypes.byref(rho) if want_rho else None)
    return st, (float(rho.value) if want_rho else None)


def jac_get_field(ctx, N: int):
    """Returns (status, N x N float32 array)."""
    out = np.empty((N, N), np.float32)
    st = load_library().jac_get_field(ctx, out.ctypes.data)
    return st, out


def jac_set_field(ctx, field) -> int:
    a = np.ascontiguousarray(field, dtype=np.float32)
    return load_library().jac_set_field(ctx, a.ctypes.data)


def jac_reset(ctx) -> int:
    return load_library().jac_reset(ctx)


def jac_fast_division(ctx) -> int:
    return load_library().jac_fast_division(ctx)


def jac_last_division(ctx) -> int:
    return load_library().jac_last_division(ctx)


def jac_depth_log(ctx):
    """Returns (status, int32 array of the depth of each check interval of the last solve)."""
    lib = load_library()
    n = ctypes.c_int64(0)
    st = lib.jac_depth_log(ctx, None, 0, ctypes.byref(n))
    if st != JAC_OK:
        return st, np.zeros(0, np.int32)
    out = np.zeros(max(n.value, 1), np.int32)
    st = lib.jac_depth_log(ctx, out.ctypes.data, int(n.value), ctypes.byref(n))
    return st, out[: n.value]


def jac_destroy(ctx) -> int:
    return load_library().jac_destroy(ctx)


def jac_profile(ctx, every: int) -> int:
    """every = 0: off; k > 0: count all launches, time every k-th of each class."""
    return load_library().jac_profile(ctx, int(every))


def jac_profile_read(ctx, kclass):
    """Returns (status, ms_timed, launches, timed_launches); kclass is an int or a KCLASS name."""
    if isinstance(kclass, str):
        kclass = KCLASS[kclass]
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    nt = ctypes.c_int64(0)
    st = load_library().jac_profile_read(ctx, int(kclass), ctypes.byref(ms), ctypes.byref(n), ctypes.byref(nt))
    return st, float(ms.value), int(n.value), int(nt.value)


def jac_stream_probe(c_ptr: int, a_ptr: int, b_ptr: int, n: int, kind: int, nontemporal: bool, blocks: int,
                     stream_ptr: int) -> int:
    """Bandwidth probe on raw device pointers: kind 0 copy, 1 add."""
    return load_library().jac_stream_probe(ctypes.c_void_p(c_ptr), ctypes.c_void_p(a_ptr),
                                           ctypes.c_void_p(b_ptr), int(n), int(kind), 1 if nontemporal else 0,
                                           int(blocks), ctypes.c_void_p(stream_ptr))


# ------------------------------------------------------------------ wrapper

def _check(st: int, allow=()):
    if st != JAC_OK and st not in allow:
        raise JacobiError(st, jac_last_error())
    return st


class Solver:
    """One libjacobi context whose workspace is a torch uint8 tensor on the GPU.

    All launches go to ``stream`` (default: torch's current stream on the
    current device).
    """

    def __init__(self, N: int, r: float, source=None, device="cuda", stream=None):
        import torch

        self.N = int(N)
        self.r = float(r)
        self.ws_bytes = jac_workspace_bytes(self.N)
        if self.ws_bytes == 0:
            raise JacobiError(JAC_EINVAL, f"N={N} out of range")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.workspace.device)
        st, h = jac_create(self.N, self.r, source, self.workspace.data_ptr(), self.ws_bytes,
                           self.stream.cuda_stream)
        _check(st)
        self.ctx = h

    def close(self):
        if getattr(self, "ctx", None):
            jac_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def solve(self, nsteps: int, opts: jac_opts | None = None, allow=()):
        opts = opts or jac_opts_default()
        st, k, rho = jac_solve(self.ctx, nsteps, opts)
        _check(st, allow)
        return st, k, rho

    def step(self, opts: jac_opts | None = None, allow=()):
        opts = opts or jac_opts_default()
        st, k, rho = jac_step(self.ctx, opts)
        _check(st, allow)
        return st, k, rho

    def sweep(self, nsweeps: int, opts: jac_opts | None = None, want_rho=False):
        opts = opts or jac_opts_default()
        st, rho = jac_sweep(self.ctx, opts, nsweeps, want_rho)
        _check(st)
        return rho

    def field(self):
        st, u = jac_get_field(self.ctx, self.N)
        _check(st)
        return u

    def set_field(self, u):
        _check(jac_set_field(self.ctx, u))

    def reset(self):
        _check(jac_reset(self.ctx))

    @property
    def fast_division(self) -> bool:
        v = jac_fast_division(self.ctx)
        if v < 0:
            _check(v)
        return bool(v)

    def depth_log(self):
        """Depth of every check interval of the most recent solve or step."""
        st, d = jac_depth_log(self.ctx)
        _check(st)
        return d

    @property
    def last_division_fast(self) -> bool:
        """True if the most recent step, sweep or solve divided by the fast path."""
        v = jac_last_division(self.ctx)
        if v < 0:
            _check(v)
        return bool(v)

    def profile(self, every: int):
        _check(jac_profile(self.ctx, every))

    def profile_read(self, kclass):
        """(average ms of the timed launches, all launches, timed launches) of a class."""
        st, ms, n, nt = jac_profile_read(self.ctx, kclass)
        _check(st)
        return (ms / nt if nt else float("nan")), n, nt
