"""Options beyond the three kernels, each bit for bit against the oracle:

* blocking checks (a standalone residual after each interval, the host decides
  before queueing more) beside the default overlapped checks -- page
  "stencil-jacobian.vercel.app", section 04, Table V (B and O);
* the unfused synchronous sweep (16 bytes per point: u^n and s read every
  sweep) -- same page, section 02 and section 05, Table VI;
* overlapping subdomains for the block-async kernel -- Islam & Wang,
  "Hierarchical Jacobi Iteration ...", sections 3.5 and 4;
* the depth controllers G-asc, G-desc and G-fb for the block-async kernel --
  same page, section 02.  G-fb decides from measured time, so its parity test
  replays the depths it chose through the oracle."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, bits, lib_solve, opts, say

pytestmark = pytest.mark.gpu

B = jac.JAC_CHECKS_BLOCKING


def solve_with_log(N, r, s, steps, o):
    sol = jac.Solver(N, r, s)
    try:
        st, k, rho = sol.solve(steps, o, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN))
        return (st, sol.field(), k, rho), sol.depth_log()
    finally:
        sol.close()


# ------------------------------------------------------------ blocking checks

@pytest.mark.parametrize("kernel,D", [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 4), (jac.JAC_TBLOCK, 8)])
@pytest.mark.parametrize("driver", [jac.JAC_LAUNCH, jac.JAC_GRAPH])
@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_blocking_checks_bitwise(kernel, D, driver, M):
    N, r = 70, 10.0
    say("blocking", kernel, D, driver, M)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=M)  # synchronous and temporal blocking: checks every M
    got, dlog = solve_with_log(N, r, s, 2, opts(kernel=kernel, D=D, M=M, driver=driver, checks=B))
    assert_same(got, ref, f"blocking {kernel} D={D} M={M}")
    assert len(dlog) == int(ref.sweeps.sum()) // M


def test_blocking_async_bitwise():
    N, r = 150, 10.0
    say("blocking async")
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=8, tx=32, ty=16)
    got, dlog = solve_with_log(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=16, checks=B))
    assert_same(got, ref, "blocking async")
    assert set(dlog.tolist()) == {8}


def test_overlapped_depth_log():
    N, r = 64, 10.0
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8)
    got, dlog = solve_with_log(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=4))
    assert_same(got, ref, "overlapped")
    assert dlog.tolist() == [4] * (int(ref.sweeps.sum()) // 8)


def test_blocking_noconv_and_nan():
    N, r = 90, 100.0
    say("blocking noconv")
    s = workloads.point_source(N, r)
    for cap in (1, 40, 41):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
        assert_same(lib_solve(N, r, s, 2, opts(checks=B, max_sweeps=cap)), ref, f"cap {cap}")
    s2 = workloads.point_source(33, 1.0)
    s2[4, 4] = np.nan
    ref = oracle.solve(33, 1.0, s2, steps=2)
    st, u, k, rho = lib_solve(33, 1.0, s2, 2, opts(checks=B))
    assert st == jac.JAC_ENAN and k.tolist() == ref.sweeps.tolist()


# ------------------------------------------------------------ unfused sweep

@pytest.mark.parametrize("N", [1, 2, 7, 70, 129, 256, 300])
@pytest.mark.parametrize("checks", [jac.JAC_CHECKS_OVERLAPPED, B])
def test_unfused_bitwise(N, checks):
    r = 10.0
    say("unfused", N, checks)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3)
    assert_same(lib_solve(N, r, s, 3, opts(kernel=jac.JAC_SYNC_UNFUSED, checks=checks)), ref, f"N={N}")


def test_unfused_graph_and_random_source():
    N, r = 130, 1.0
    say("unfused graph")
    s = workloads.random_source(N, r, 7)
    u0 = workloads.random_field(N, 8)
    ref = oracle.solve(N, r, s, u0=u0, steps=3)
    assert_same(lib_solve(N, r, s, 3, opts(kernel=jac.JAC_SYNC_UNFUSED, driver=jac.JAC_GRAPH), u0=u0), ref,
                "unfused graph")


def test_unfused_not_persistent():
    sol = jac.Solver(16, 1.0)
    try:
        st, _, _ = jac.jac_step(sol.ctx, opts(kernel=jac.JAC_SYNC_UNFUSED, driver=jac.JAC_PERSISTENT))
        assert st == jac.JAC_EINVAL
    finally:
        sol.close()


# ------------------------------------------------------------ overlap

@pytest.mark.parametrize("tile,D,o", [((32, 8), 8, 1), ((32, 8), 8, 2), ((16, 16), 4, 1), ((7, 5), 3, 2),
                                      ((32, 16), 8, 4), ((64, 16), 6, 3)])
def test_overlap_bitwise(tile, D, o):
    N, r = 150, 10.0
    say("overlap", tile, D, o)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1], o=o)
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=tile[0], tile_y=tile[1], overlap=o))
    assert_same(got, ref, f"{tile} D={D} o={o}")


@pytest.mark.parametrize("D", [2, 5, 8])
def test_overlap_at_least_depth_is_sync(D):
    """o >= D - 1: no stale value reaches a tile's own points, so the
    block-async solve is the synchronous solve exactly."""
    N, r = 97, 10.0
    say("overlap exact", D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8)
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=16, tile_y=8, overlap=D - 1))
    assert_same(got, ref, f"D={D}")


def test_overlap_graph_driver():
    N, r = 120, 10.0
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=8, tx=32, ty=8, o=2)
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=8, overlap=2,
                                     driver=jac.JAC_GRAPH))
    assert_same(got, ref, "graph o=2")


def test_overlap_rejections():
    sol = jac.Solver(32, 1.0)
    try:
        for o in (opts(kernel=jac.JAC_ASYNC, D=4, tile_x=64, tile_y=64, overlap=1),   # region > 4096
                  opts(kernel=jac.JAC_ASYNC, D=4, overlap=65),
                  opts(kernel=jac.JAC_ASYNC, D=4, overlap=-1),
                  opts(kernel=jac.JAC_TBLOCK, D=4, overlap=1),
                  opts(kernel=jac.JAC_ASYNC, D=4, overlap=1, driver=jac.JAC_PERSISTENT)):
            assert jac.jac_step(sol.ctx, o)[0] == jac.JAC_EINVAL
    finally:
        sol.close()


# ------------------------------------------------------------ controllers

@pytest.mark.parametrize("ctrl,oc", [(jac.JAC_G_ASC, oracle.G_ASC), (jac.JAC_G_DESC, oracle.G_DESC)])
@pytest.mark.parametrize("r,D", [(10.0, 8), (100.0, 8), (10.0, 4), (10.0, 6), (100.0, 6), (10.0, 16)])
def test_threshold_controllers_bitwise(ctrl, oc, r, D):
    """The capped levels min(level, D): D = 4 and 6 below the top level, 16 above it."""
    N = 64
    say("controller", ctrl, r, D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=D, tx=32, ty=8, controller=oc,
                       log_cap=100000)
    got, dlog = solve_with_log(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=32, tile_y=8, controller=ctrl))
    assert_same(got, ref, f"ctrl {ctrl} r={r}")
    assert dlog.tolist() == ref.D_log.tolist()


@pytest.mark.parametrize("r", [10.0, 100.0])
def test_feedback_controller_replays_in_oracle(r):
    """G-fb picks depths from measured time; whatever it picked, the same
    schedule through the oracle gives the same solve bit for bit."""
    N = 96
    say("G-fb", r)
    s = workloads.gaussian_source(N, r)
    got, dlog = solve_with_log(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=8,
                                                controller=jac.JAC_G_FB))
    assert set(dlog.tolist()) <= {1, 2, 4, 8} and dlog[0] == 1
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=8, tx=32, ty=8, controller=oracle.SCHED,
                       schedule=dlog, log_cap=100000)
    assert_same(got, ref, f"G-fb r={r}")
    assert np.all(got[3] < 1e-5)


def test_controller_rejections():
    sol = jac.Solver(32, 1.0)
    try:
        for o in (opts(kernel=jac.JAC_TBLOCK, D=4, controller=jac.JAC_G_ASC),
                  opts(kernel=jac.JAC_ASYNC, D=8, controller=jac.JAC_G_ASC, driver=jac.JAC_GRAPH),
                  opts(kernel=jac.JAC_ASYNC, D=8, controller=7),
                  opts(checks=5)):
            assert jac.jac_step(sol.ctx, o)[0] == jac.JAC_EINVAL
    finally:
        sol.close()
