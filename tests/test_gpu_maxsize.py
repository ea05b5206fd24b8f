"""The library's largest grid, N = 65536: 4.3 G unknowns, a padded plane of
more than 2^32 floats (17 GB) and a 64.5 GiB workspace, so every global
offset has to be 64-bit.

The oracle cannot solve that grid, so the check uses a property that holds at
any size.  From u = 0 under a constant source, a point's value after k sweeps
depends only on the points within k cells of it (block-async: within D + 1
cells per launch, and on where the point sits in its tile, since tile edges
hold frozen halos).  Away from the boundary the iterate is therefore periodic:
period 1 for the exact sweeps, the tile's 16 rows x 32 columns for block-async
tiles of 32 x 16.  A 96 x 96 grid solved by the oracle holds every value the
big grid can take: its first and last 32 rows and columns are the big grid's,
and each interior point of the big grid takes the value of the small grid's
interior point with the same phase in the period.  The maxima that form rho
(the residual's and ||b_A||'s) range over the same set of values on both
grids, so sweeps, status and rho agree too (page "stencil-jacobian.vercel.app",
section 01: the five-point backward-Euler step and its rho test).
"""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
from tests.gpu_helpers import bits, opts, say

N_MAX = 65536
N_SMALL = 96
EDGE = 32      # rows and columns next to the boundary that are mapped one to one
R = 10.0
C = np.float32(0.25)
CAP = 24       # sweeps: three checks every 8; influence reaches at most 27 cells

TB = jac.JAC_TBLOCK
CASES = {
    "sync": dict(kernel=jac.JAC_SYNC, D=1, period=(1, 1)),
    "tblock D11": dict(kernel=TB, D=11, period=(1, 1)),
    "tblock D4": dict(kernel=TB, D=4, period=(1, 1)),
    "async D8 32x16": dict(kernel=jac.JAC_ASYNC, D=8, tile=(32, 16), period=(16, 32)),
}


def small_index(n_big, period):
    """Index into the small grid for each row (or column) of the big grid."""
    idx = np.empty(n_big, np.int64)
    idx[:EDGE] = np.arange(EDGE)
    idx[n_big - EDGE:] = np.arange(N_SMALL - EDGE, N_SMALL)
    mid = np.arange(EDGE, n_big - EDGE)
    idx[EDGE:n_big - EDGE] = EDGE + (mid - EDGE) % period
    return idx


def oracle_small(case):
    c = CASES[case]
    s = np.full((N_SMALL, N_SMALL), C, np.float32)
    if c["kernel"] == jac.JAC_ASYNC:
        tx, ty = c["tile"]
        return oracle.solve(N_SMALL, R, s, steps=1, M=8, mode=oracle.ASYNC, D=c["D"], tx=tx, ty=ty,
                            max_sweeps=CAP)
    return oracle.solve(N_SMALL, R, s, steps=1, M=8, max_sweeps=CAP)


def assert_periodic_image(got, ref_u, period, label, chunk=1024):
    """got (n x n) must equal the small field mapped through small_index, row block by row block."""
    n = got.shape[0]
    ri = small_index(n, period[0])
    ci = small_index(n, period[1])
    cols = ref_u[:, ci]                       # N_SMALL x n
    for r0 in range(0, n, chunk):
        want = cols[ri[r0:r0 + chunk]]
        assert np.array_equal(bits(got[r0:r0 + chunk]), bits(want)), f"{label}: rows {r0}..{r0 + chunk - 1}"


@pytest.mark.parametrize("case", sorted(CASES))
def test_periodic_image_holds_in_the_oracle(case):
    """The mapping itself, on the CPU: a 480 x 480 oracle grid (a multiple of
    both periods, like 65536) is the 96 x 96 one mapped, bit for bit, with the
    same sweeps and rho."""
    c = CASES[case]
    ref = oracle_small(case)
    n = 480
    s = np.full((n, n), C, np.float32)
    if c["kernel"] == jac.JAC_ASYNC:
        tx, ty = c["tile"]
        big = oracle.solve(n, R, s, steps=1, M=8, mode=oracle.ASYNC, D=c["D"], tx=tx, ty=ty, max_sweeps=CAP)
    else:
        big = oracle.solve(n, R, s, steps=1, M=8, max_sweeps=CAP)
    assert ref.status == big.status == oracle.ENOCONV
    assert ref.sweeps.tolist() == big.sweeps.tolist() == [CAP]
    assert bits(ref.rho).tolist() == bits(big.rho).tolist()
    assert_periodic_image(big.u, ref.u, c["period"], case, chunk=100)


@pytest.fixture(scope="module")
def big_solver():
    import psutil
    import torch
    ws = jac.jac_workspace_bytes(N_MAX)
    free, _ = torch.cuda.mem_get_info()
    if free < ws + (4 << 30):
        pytest.skip(f"N = {N_MAX} needs {ws / 2**30:.1f} GiB of device memory, {free / 2**30:.1f} free")
    if psutil.virtual_memory().available < (48 << 30):
        pytest.skip("N = 65536 needs about 40 GiB of host memory for the source and the field")
    say("max size: create", N_MAX)
    sol = jac.Solver(N_MAX, R, np.full((N_MAX, N_MAX), C, np.float32))
    yield sol
    sol.close()
    sol.workspace = None      # the fixture's cached value still refers to sol
    torch.cuda.empty_cache()  # hand the 64.5 GiB back for the tests that follow


@pytest.mark.gpu
@pytest.mark.parametrize("case", sorted(CASES))
def test_maximum_grid_bitwise(case, big_solver):
    """N = 65536, r = 10, constant source, one step capped at 24 sweeps (three
    checks every 8): status, sweeps, rho bits and all 4.3 G values against the
    96 x 96 oracle grid mapped as above."""
    c = CASES[case]
    ref = oracle_small(case)
    assert ref.status == oracle.ENOCONV and ref.sweeps[0] == CAP
    say("max size", N_MAX, case)
    sol = big_solver
    sol.reset()
    tx, ty = c.get("tile", (32, 8))
    st, k, rho = sol.step(opts(kernel=c["kernel"], D=c["D"], tile_x=tx, tile_y=ty, max_sweeps=CAP),
                          allow=(jac.JAC_ENOCONV,))
    assert st == jac.JAC_ENOCONV and k == CAP, (st, k)
    assert np.float32(rho).view(np.uint32) == ref.rho[0].view(np.uint32), (rho, ref.rho[0])
    say("max size: compare", case)
    assert_periodic_image(sol.field(), ref.u, c["period"], case)
