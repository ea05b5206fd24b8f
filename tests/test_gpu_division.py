"""The sweep's division by d = 1 + 4r.  A context divides through RN(1/d) and one
fma correction only after a set-up kernel has found it equal to the IEEE
quotient on every float input other than Inf, NaN and -0, and a step takes
that path only when the host can rule those numerators out; every path must
give the oracle's results."""
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
    sol = jac.Solver(8, r, workloads.gaussian_source(8, r))
    try:
        assert sol.fast_division
        assert not sol.last_division_fast  # no work yet
        sol.step(opts())
        assert sol.last_division_fast
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


@pytest.mark.parametrize("kernel,D", [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 8)])
def test_negative_zero_source_takes_ieee_division(kernel, D):
    """A -0 in the source could make a numerator -0, which the fast quotient
    maps to +0: such a context divides by IEEE division."""
    N, r = 65, 10.0
    say("division -0", kernel)
    s = workloads.gaussian_source(N, r)
    s[0, 5] = np.float32(-0.0)
    s[40, 40] = np.float32(-0.0)
    sol = jac.Solver(N, r, s)
    try:
        st, k, rho = sol.solve(2, opts(kernel=kernel, D=D))
        assert sol.fast_division and not sol.last_division_fast
        u = sol.field()
    finally:
        sol.close()
    assert_same((st, u, k, rho), oracle.solve(N, r, s, steps=2), "-0 source")


@pytest.mark.parametrize("driver", [jac.JAC_LAUNCH, jac.JAC_GRAPH])
def test_bound_near_overflow_switches_to_ieee(driver):
    """A source of 1e37: the carried bound on |u| grows by max|s| per step, so
    the first steps divide by the fast path and later ones, whose numerators
    the bound can no longer keep finite, by IEEE division.  Every step matches
    the oracle bit for bit (the field itself stays finite)."""
    N, r, steps = 8, 1.0, 8
    say("division bound", driver)
    s = np.full((N, N), 1e37, np.float32)
    ref = oracle.solve(N, r, s, steps=steps)
    sol = jac.Solver(N, r, s)
    paths, ks, rhos = [], [], []
    try:
        for _ in range(steps):
            st, k, rho = sol.step(opts(driver=driver))
            assert st == jac.JAC_OK
            paths.append(sol.last_division_fast)
            ks.append(k)
            rhos.append(rho)
        u = sol.field()
        assert paths[0] and not paths[-1], paths
        assert paths == sorted(paths, reverse=True), paths
        assert ks == ref.sweeps.tolist()
        assert np.array_equal(np.array(rhos, np.float32).view(np.uint32), ref.rho.view(np.uint32))
        assert np.array_equal(u.view(np.uint32), ref.u.view(np.uint32))
        assert np.isfinite(u).all()
        sol.reset()  # the bound restarts from u = 0
        sol.step(opts(driver=driver))
        assert sol.last_division_fast
    finally:
        sol.close()


def test_set_field_with_infinity_takes_ieee_division():
    N, r = 33, 10.0
    say("division set_field inf")
    s = workloads.gaussian_source(N, r)
    u0 = np.zeros((N, N), np.float32)
    u0[3, 3] = np.inf
    sol = jac.Solver(N, r, s)
    try:
        sol.set_field(u0)
        st, k, rho = sol.step(opts(max_sweeps=16), allow=(jac.JAC_ENAN, jac.JAC_ENOCONV))
        assert not sol.last_division_fast
        u = sol.field()
        sol.set_field(np.zeros((N, N), np.float32))
        sol.step(opts())
        assert sol.last_division_fast
    finally:
        sol.close()
    ref = oracle.solve(N, r, s, u0=u0, steps=1, max_sweeps=16)
    assert st == ref.status and [k] == ref.sweeps.tolist()
    assert np.array_equal(np.isnan(u), np.isnan(ref.u)) and np.array_equal(np.isinf(u), np.isinf(ref.u))
    fin = np.isfinite(ref.u)
    assert np.array_equal(u[fin].view(np.uint32), ref.u[fin].view(np.uint32))
