"""Temporal blocking deeper than the check interval (D = 9..16 over checks
every M sweeps), through the launch driver: a launch of up to D sweeps measures
the residual of the levels where checks fall, at most two per launch.  A check
that stops the step at an inner level leaves its iterate unstored, so a redo
launch recomputes it from the launch's intact input; a launch ends on a check
predicted to stop, which then runs as a residual pass on the exact iterate.
Whatever the schedule, the result is the oracle's with checks every M sweeps
(page "stencil-jacobian.vercel.app", section 01: rho checked every M = 8
sweeps; section 02: D sweeps of temporal blocking equal D synchronous sweeps)."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, opts, say

pytestmark = pytest.mark.gpu

TB = jac.JAC_TBLOCK


def solve_profiled(N, r, s, steps, o, u0=None):
    """(status, field, sweeps, rho) and the launch counts per class."""
    sol = jac.Solver(N, r, s)
    try:
        if u0 is not None:
            sol.set_field(u0)
        sol.profile(1)
        st, k, rho = sol.solve(steps, o, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN))
        u = sol.field()
        n = {c: sol.profile_read(c)[1] for c in ("tblock", "tblock_part", "residual", "tblock_rhs")}
    finally:
        sol.close()
    return (st, u, k, rho), n


@pytest.mark.parametrize("margin", ["0", None, "1e30"])
@pytest.mark.parametrize("M", [8, 5])
@pytest.mark.parametrize("D", list(range(9, 17)))
def test_deep_launches_bitwise(D, M, margin, monkeypatch):
    """Every depth over checks every 8 and every 5 sweeps, with prediction off
    (stops land inside launches: redo launches; row-sampled checks off too, so
    that no check is measured twice), at its default and forced at every check
    (launches end on each predicted check, most predictions fail)."""
    if margin is None:
        monkeypatch.delenv("JACOBI_PREDICT_MARGIN", raising=False)
    else:
        monkeypatch.setenv("JACOBI_PREDICT_MARGIN", margin)
    if margin == "0":
        monkeypatch.setenv("JACOBI_SAMPLED_CHECKS", "0")
    else:
        monkeypatch.delenv("JACOBI_SAMPLED_CHECKS", raising=False)
    N, r = 150, 10.0
    say("deep", D, M, margin)
    s = workloads.random_source(N, r, 31)
    u0 = workloads.random_field(N, 31)
    ref = oracle.solve(N, r, s, u0=u0, steps=3, M=M)
    res, n = solve_profiled(N, r, s, 3, opts(kernel=TB, D=D, M=M), u0=u0)
    assert_same(res, ref, f"D={D} M={M} margin={margin}")
    # launches of D sweeps, or of 2M + c when two checks already fall inside
    assert n["tblock"] + n["tblock_part"] > 0
    if 2 * M >= D:
        assert n["tblock"] > 0
    if margin == "0":
        assert n["residual"] == 0
    elif margin == "1e30":
        assert n["residual"] >= 3


@pytest.mark.parametrize("D,M", [(12, 3), (16, 1), (9, 4), (16, 7)])
def test_deep_small_intervals_bitwise(D, M):
    """Short intervals: launches hold at most two checks, and launches of 8
    sweeps or fewer check only their input."""
    N, r = 70, 1.0
    say("deep small M", D, M)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=M)
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=D, M=M))
    assert_same(res, ref, f"D={D} M={M}")


@pytest.mark.parametrize("cap", [40, 44, 45, 8, 1])
@pytest.mark.parametrize("margin", ["0", "1e30"])
def test_deep_sweep_cap_and_nan(cap, margin, monkeypatch):
    """A sweep cap ends the step on the first check at or past it (launches
    never run past that check), and a NaN ends it with the oracle's field."""
    monkeypatch.setenv("JACOBI_PREDICT_MARGIN", margin)
    N, r = 97, 10.0
    say("deep cap/nan", cap, margin)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
    assert ref.status == oracle.ENOCONV
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, max_sweeps=cap))
    assert_same(res, ref, f"cap {cap}")
    u0 = np.zeros((N, N), np.float32)
    u0[N // 3, N // 2] = np.inf
    ref = oracle.solve(N, r, s, u0=u0, steps=2)
    assert ref.status == oracle.ENAN
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=13), u0=u0)
    assert_same(res, ref, "nan")


@pytest.mark.parametrize("D", [10, 16])
def test_deep_ieee_division_bitwise(D, monkeypatch):
    """With IEEE division the step keeps the separate right-hand-side pass in
    front of the deep launches."""
    monkeypatch.setenv("JACOBI_IEEE_DIVISION", "1")
    N, r = 120, 100.0
    say("deep ieee", D)
    s = workloads.random_source(N, r, 5)
    ref = oracle.solve(N, r, s, steps=2)
    res, n = solve_profiled(N, r, s, 2, opts(kernel=TB, D=D))
    assert_same(res, ref, f"ieee D={D}")
    assert n["tblock_rhs"] == 0


def test_deep_band_heights_and_graph_and_blocking_bitwise():
    """Tall and short bands under deep launches; the graph driver and blocking
    checks with D above M launch M sweeps at a time -- all on the oracle's bits."""
    N, r = 300, 10.0
    say("deep bands/graph/blocking")
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8)
    for H in (4, 64, 300):
        res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, band_rows=H))
        assert_same(res, ref, f"H={H}")
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, driver=jac.JAC_GRAPH))
    assert_same(res, ref, "graph")
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, checks=jac.JAC_CHECKS_BLOCKING))
    assert_same(res, ref, "blocking")
    res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, driver=jac.JAC_PERSISTENT))
    assert_same(res, ref, "persistent")


@pytest.mark.parametrize("D,M", [(11, 8), (9, 8), (12, 8), (16, 5)])
def test_sampled_checks_bitwise(D, M, monkeypatch):
    """A check that is not expected to stop measures the residual on every
    8th row: that maximum bounds R from below, so a sample at or above tol
    decides the check exactly, and a sample below tol is measured again in
    full before the step stops or goes on.  With only row 0 sampled (stride
    2^20) many late checks are measured twice, and the step goes on from the
    checked iterate; with sampling off every check measures every row.  All
    three give the oracle's sweeps, rho and field bit for bit."""
    N, r = 300, 10.0
    s = workloads.gaussian_source(N, r)
    u0 = workloads.random_field(N, 7)
    ref = oracle.solve(N, r, s, u0=u0, steps=3, M=M)
    runs = {}
    for stride in ("0", "8", "1048576"):
        monkeypatch.setenv("JACOBI_SAMPLED_CHECKS", stride)
        say("deep sampled", D, M, stride)
        res, n = solve_profiled(N, r, s, 3, opts(kernel=TB, D=D, M=M), u0=u0)
        assert_same(res, ref, f"D={D} M={M} stride={stride}")
        runs[stride] = n
    # every sample below tol is measured again by a residual pass of its own
    assert runs["1048576"]["residual"] > runs["0"]["residual"]


def test_sampled_checks_c3_shape(monkeypatch):
    """N = 1024, r = 10, the benchmark's depth and interval: sampled checks
    (the default) against sampling off, both the oracle's bits."""
    N, r = 1024, 10.0
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8)
    for stride in ("8", "0"):
        monkeypatch.setenv("JACOBI_SAMPLED_CHECKS", stride)
        say("deep sampled N=1024", stride)
        res, _ = solve_profiled(N, r, s, 2, opts(kernel=TB, D=11, M=8))
        assert_same(res, ref, f"stride={stride}")
