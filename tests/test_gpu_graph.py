"""The graph driver: each check interval is captured once as a HIP graph and
replayed (the launch-bound regime of page "cuda-solver-lab", where a CUDA Graph
cut the time per iteration at 256^2).  Replays must give the oracle's results
bit for bit, also when eager launches of the same context run between them."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, bits, lib_solve, opts, say

pytestmark = pytest.mark.gpu

GR = jac.JAC_GRAPH


@pytest.mark.parametrize("kernel,D,M", [(jac.JAC_SYNC, 1, 8), (jac.JAC_SYNC, 1, 3), (jac.JAC_TBLOCK, 3, 8),
                                        (jac.JAC_TBLOCK, 8, 8), (jac.JAC_TBLOCK, 5, 5)])
@pytest.mark.parametrize("N", [7, 70, 257])
def test_graph_bitwise(kernel, D, M, N):
    r = 10.0
    say("graph", kernel, D, M, N)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3, M=max(M, D))
    assert_same(lib_solve(N, r, s, 3, opts(kernel=kernel, D=D, M=M, driver=GR)), ref, f"{kernel} D={D} M={M}")


def test_graph_async_bitwise():
    N, r = 150, 10.0
    say("graph async")
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=8, tx=32, ty=16)
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=16, driver=GR))
    assert_same(got, ref, "async")


@pytest.mark.parametrize("r", [1.0, 10.0])
def test_config_c5_bitwise(r):
    say("graph C5", r)
    s = workloads.gaussian_source(256, r)
    ref = oracle.solve(256, r, s)
    assert_same(lib_solve(256, r, s, 10, opts(driver=GR)), ref, f"C5 r={r}")


def test_replays_interleaved_with_eager_work():
    """Graph solves, eager solves and option changes on one context; every
    replay is checked against the oracle."""
    N, r = 129, 10.0
    say("graph interleaved")
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2)
    ref_tb = oracle.solve(N, r, s, steps=2, M=8)
    sol = jac.Solver(N, r, s)
    try:
        for rep in range(4):
            for o, want in ((opts(driver=GR), ref), (opts(), ref), (opts(kernel=jac.JAC_TBLOCK, D=4, driver=GR),
                                                                     ref_tb)):
                sol.reset()
                st, k, rho = sol.solve(2, o)
                u = sol.field()
                assert k.tolist() == want.sweeps.tolist(), (rep, o.driver, o.kernel)
                assert np.array_equal(bits(u), bits(want.u)), (rep, o.driver, o.kernel)
                assert np.array_equal(bits(rho), bits(want.rho))
    finally:
        sol.close()


def test_graph_noconv_and_nan():
    N, r = 90, 100.0
    say("graph noconv")
    s = workloads.point_source(N, r)
    for cap in (1, 40, 41):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
        assert_same(lib_solve(N, r, s, 2, opts(driver=GR, max_sweeps=cap)), ref, f"cap {cap}")
    s2 = workloads.point_source(33, 1.0)
    s2[4, 4] = np.nan
    ref = oracle.solve(33, 1.0, s2, steps=2)
    st, u, k, rho = lib_solve(33, 1.0, s2, 2, opts(driver=GR))
    assert st == jac.JAC_ENAN and k.tolist() == ref.sweeps.tolist()
