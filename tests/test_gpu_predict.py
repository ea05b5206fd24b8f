"""Final-check prediction with overlapped checks: a check whose rho the last
checks extrapolate below the tolerance runs as a residual pass alone, and a
check that then does not converge is followed by the interval it skipped.
Results must equal the oracle's bit for bit whatever the prediction does
(page "stencil-jacobian.vercel.app", section 02: identical sweep counts for
every kernel).  The margin is read from JACOBI_PREDICT_MARGIN at create time:
a huge margin predicts at every check once three are known, so most
predictions fail and the recovery path runs; 0 turns prediction off."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, opts, say

pytestmark = pytest.mark.gpu

TB, ASYNC = jac.JAC_TBLOCK, jac.JAC_ASYNC
CASES = [(jac.JAC_SYNC, 1, jac.JAC_LAUNCH), (TB, 8, jac.JAC_LAUNCH), (TB, 4, jac.JAC_GRAPH),
         (jac.JAC_SYNC, 1, jac.JAC_GRAPH)]


def solve_counting(N, r, s, steps, o, u0=None):
    sol = jac.Solver(N, r, s)
    try:
        if u0 is not None:
            sol.set_field(u0)
        sol.profile(1)
        st, k, rho = sol.solve(steps, o, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN))
        u = sol.field()
        _, n_resid, _ = sol.profile_read("residual")
    finally:
        sol.close()
    return (st, u, k, rho), n_resid


@pytest.mark.parametrize("margin", ["1e30", None, "0"])
@pytest.mark.parametrize("kernel,D,driver", CASES)
def test_prediction_keeps_oracle_bits(kernel, D, driver, margin, monkeypatch):
    if margin is None:
        monkeypatch.delenv("JACOBI_PREDICT_MARGIN", raising=False)
    else:
        monkeypatch.setenv("JACOBI_PREDICT_MARGIN", margin)
    # with the prediction off, no residual pass of its own may run: row-sampled
    # checks (whose samples below tol are measured again in full) off as well
    if margin == "0":
        monkeypatch.setenv("JACOBI_SAMPLED_CHECKS", "0")
    else:
        monkeypatch.delenv("JACOBI_SAMPLED_CHECKS", raising=False)
    N, r = 150, 10.0
    say("predict", kernel, D, driver, margin)
    s = workloads.random_source(N, r, 21)
    u0 = workloads.random_field(N, 21)
    ref = oracle.solve(N, r, s, u0=u0, steps=3)
    res, n_resid = solve_counting(N, r, s, 3, opts(kernel=kernel, D=D, driver=driver), u0=u0)
    assert_same(res, ref, f"kernel {kernel} D {D} driver {driver} margin {margin}")
    if margin == "0":
        assert n_resid == 0
    elif margin == "1e30":
        assert n_resid >= 3  # every step predicts from its fourth check on


def test_prediction_with_max_sweeps_and_async(monkeypatch):
    """A cap that ends the step between predictions, and the block-async kernel
    (its own sweep counts), under forced predictions."""
    monkeypatch.setenv("JACOBI_PREDICT_MARGIN", "1e30")
    N, r = 97, 10.0
    say("predict cap/async")
    s = workloads.gaussian_source(N, r)
    for cap in (40, 48, 56):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
        res, _ = solve_counting(N, r, s, 2, opts(kernel=TB, D=8, max_sweeps=cap))
        assert_same(res, ref, f"cap {cap}")
    ref = oracle.solve(N, r, s, steps=3, mode=oracle.ASYNC, D=4, tx=32, ty=8)
    res, n_resid = solve_counting(N, r, s, 3, opts(kernel=ASYNC, D=4, tile_x=32, tile_y=8))
    assert_same(res, ref, "async D4 32x8")
    assert n_resid >= 3
