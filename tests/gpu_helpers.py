"""Shared helpers for the GPU tests: run the library through its C interface and
compare with the oracle bit for bit."""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

import jacobi_stencil_amd as jac

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*args):
    """Name the case before it runs, so a failing GPU run still says which."""
    print("[case]", *args, file=sys.stderr, flush=True)


def opts(kernel=jac.JAC_SYNC, driver=jac.JAC_LAUNCH, D=1, tile_x=32, tile_y=8, M=8, tol=1e-5,
         max_sweeps=10**6, band_rows=0, checks=jac.JAC_CHECKS_OVERLAPPED, controller=jac.JAC_STATIC, overlap=0):
    return jac.jac_opts_default(kernel=kernel, driver=driver, D=D, tile_x=tile_x, tile_y=tile_y, M=M,
                                tol=tol, max_sweeps=max_sweeps, band_rows=band_rows, checks=checks,
                                controller=controller, overlap=overlap)


def lib_solve(N, r, s, steps, o, u0=None, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN)):
    """Returns (status, field, sweeps, rho) from the library."""
    sol = jac.Solver(N, r, s)
    try:
        if u0 is not None:
            sol.set_field(u0)
        st, k, rho = sol.solve(steps, o, allow=allow)
        return st, sol.field(), k, rho
    finally:
        sol.close()


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def assert_same(lib, orc_res, what=""):
    st, u, k, rho = lib
    assert st == orc_res.status, f"{what}: status {st} vs oracle {orc_res.status}"
    assert k.tolist() == orc_res.sweeps.tolist(), f"{what}: sweeps {k.tolist()} vs {orc_res.sweeps.tolist()}"
    assert np.array_equal(bits(rho), bits(orc_res.rho)), f"{what}: rho {rho} vs {orc_res.rho}"
    if not np.array_equal(bits(u), bits(orc_res.u)):
        diff = np.argwhere(bits(u) != bits(orc_res.u))
        i, j = diff[0]
        raise AssertionError(f"{what}: {len(diff)} points differ, first at ({i},{j}): "
                             f"{u[i, j]!r} vs {orc_res.u[i, j]!r}")


def field_hash(u) -> str:
    return hashlib.sha256(np.ascontiguousarray(u, dtype="<f4").tobytes()).hexdigest()


def load_expected(name):
    path = os.path.join(GOLDEN, f"expected_{name}.json")
    if not os.path.exists(path):
        return None
    return json.load(open(path))
