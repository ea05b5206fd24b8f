"""jac_sweep_static -- jac_sweep with the library's static device scratch, for
callers that cannot allocate -- against jac_sweep itself, bit for bit: the
field, and rho of the last iterate, over two calls in a row on one context,
then again on a smaller grid (the static array keeps the previous call's
contents, which must not leak into the next)."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import workloads
from tests.gpu_helpers import bits, say

pytestmark = pytest.mark.gpu

CASES = [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 8), (jac.JAC_ASYNC, 4), (jac.JAC_SYNC_UNFUSED, 1)]


def _two_calls(N, r, kernel, D, nsweeps, static):
    sol = jac.Solver(N, r, workloads.gaussian_source(N, r))
    try:
        o = jac.jac_opts_default(kernel=kernel, D=D, tile_x=32, tile_y=8)
        fn = jac.jac_sweep_static if static else jac.jac_sweep
        out = []
        for n in (nsweeps, nsweeps // 2 + 1):  # the second call starts from the first one's field
            st, rho = fn(sol.ctx, o, n, True)
            assert st == jac.JAC_OK, jac.jac_last_error()
            out.append(rho)
        return sol.field(), np.array(out, np.float32)
    finally:
        sol.close()


@pytest.mark.parametrize("kernel,D", CASES)
def test_static_scratch_matches_jac_sweep(kernel, D):
    for N, nsw in ((700, 37), (90, 21)):  # then a smaller grid
        say("jac_sweep_static", kernel, D, N)
        u_ref, rho_ref = _two_calls(N, 10.0, kernel, D, nsw, static=False)
        u, rho = _two_calls(N, 10.0, kernel, D, nsw, static=True)
        assert np.array_equal(bits(rho), bits(rho_ref)), (rho, rho_ref)
        assert np.array_equal(bits(u), bits(u_ref)), f"N={N}: field differs"


def test_static_and_workspace_calls_interleave():
    """Static-scratch and workspace-scratch sweeps alternate on one context and
    give what workspace-scratch sweeps alone give."""
    N, r = 300, 10.0
    say("jac_sweep_static interleaved")
    o = jac.jac_opts_default(kernel=jac.JAC_TBLOCK, D=4)
    res = []
    for static_first in (False, True):
        sol = jac.Solver(N, r, workloads.gaussian_source(N, r))
        try:
            rhos = []
            for k in range(4):
                fn = jac.jac_sweep_static if (k % 2 == 0) == static_first else jac.jac_sweep
                st, rho = fn(sol.ctx, o, 13, True)
                assert st == jac.JAC_OK, jac.jac_last_error()
                rhos.append(rho)
            res.append((sol.field(), np.array(rhos, np.float32)))
        finally:
            sol.close()
    assert np.array_equal(bits(res[0][1]), bits(res[1][1]))
    assert np.array_equal(bits(res[0][0]), bits(res[1][0]))


def test_static_scratch_limit():
    """Above N = 16384 the call is refused before anything runs."""
    N = 16385
    say("jac_sweep_static limit")
    sol = jac.Solver(N, 1.0)
    try:
        st, _ = jac.jac_sweep_static(sol.ctx, jac.jac_opts_default(), 8, True)
        assert st == jac.JAC_EINVAL and "16384" in jac.jac_last_error()
        assert not np.any(sol.field()[:4])  # the field is still u^0 = 0
    finally:
        sol.close()
