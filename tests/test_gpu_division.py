"""The sweep's division by d = 1 + 4r.  A context divides through RN(1/d) and one
fma correction only after a set-up kernel has found it equal to the IEEE
quotient on every float input; both paths must give the oracle's results."""
import os

import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, lib_solve, opts, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("r", [1.0, 10.0, 100.0])
def test_fast_division_verified_for_the_measured_couplings(r):
    """d = 5, 41, 401: the exhaustive check passes (also checked on the CPU for
    these d against x86 division), so the measured workloads use the fast path."""
    say("division flag", r)
    sol = jac.Solver(8, r)
    try:
        assert sol.fast_division
    finally:
        sol.close()


@pytest.mark.parametrize("r", [0.0, 0.25, 0.1, 3.7, 1234.5])
def test_other_couplings_are_exact_either_way(r):
    """Whatever path the check picks, results match the oracle bit for bit."""
    N = 65
    say("division other r", r)
    s = workloads.random_source(N, max(r, 1.0), 3) + np.float32(0.5)
    ref = oracle.solve(N, r, s, steps=2)
    assert_same(lib_solve(N, r, s, 2, opts()), ref, f"sync r={r}")
    assert_same(lib_solve(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=4)), ref, f"tblock r={r}")


@pytest.mark.parametrize("kernel,D", [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 8)])
def test_ieee_division_path_bitwise(kernel, D, monkeypatch):
    N, r = 129, 10.0
    say("division ieee", kernel, D)
    monkeypatch.setenv("JACOBI_IEEE_DIVISION", "1")
    s = workloads.gaussian_source(N, r)
    sol = jac.Solver(N, r, s)
    try:
        assert not sol.fast_division
        st, k, rho = sol.solve(3, opts(kernel=kernel, D=D))
        u = sol.field()
    finally:
        sol.close()
    ref = oracle.solve(N, r, s, steps=3)
    assert_same((st, u, k, rho), ref, "ieee path")
