"""The persistent driver: the whole solve in one cooperative kernel with the
residual, the decision and the time loop on the device (page "stencil-jacobian.
vercel.app", section 04, the host round trip as the cost to remove; the
CPU-free model of the arXiv 2610.15878 summary).  Results must equal the
oracle's exactly as with per-launch issue: SYNC and TBLOCK bit for bit with the
synchronous oracle, ASYNC with the oracle's block-async model."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, field_hash, lib_solve, load_expected, opts, say

pytestmark = pytest.mark.gpu

PER = jac.JAC_PERSISTENT


@pytest.mark.parametrize("N", [1, 2, 3, 7, 33, 64, 65, 70, 129, 256, 257, 300])
def test_sync_small_grids_bitwise(N):
    r = 10.0
    say("persist sync", N)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3)
    assert_same(lib_solve(N, r, s, 3, opts(driver=PER)), ref, f"N={N}")


@pytest.mark.parametrize("D", list(range(1, 17)))
def test_tblock_every_depth_bitwise(D):
    N, r = 150, 10.0
    say("persist tblock", D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=max(8, D))
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=D, M=max(8, D), driver=PER))
    assert_same(got, ref, f"D={D}")


@pytest.mark.parametrize("tile,D", [((32, 8), 8), ((32, 16), 8), ((7, 5), 3), ((64, 16), 12)])
def test_async_bitwise(tile, D):
    N, r = 150, 10.0
    say("persist async", tile, D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1])
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=tile[0], tile_y=tile[1], driver=PER))
    assert_same(got, ref, f"{tile} D={D}")


@pytest.mark.parametrize("N,tile,D", [(256, (32, 16), 8), (256, (32, 8), 4), (33, (32, 8), 8), (150, (64, 16), 12),
                                      (1, (32, 8), 8), (2, (32, 16), 3), (97, (16, 16), 1), (300, (64, 60), 6),
                                      (130, (1, 64), 5), (150, (7, 5), 3), (1024, (32, 16), 8), (700, (32, 8), 4),
                                      (1000, (16, 16), 3), (1500, (64, 64), 2)])
def test_async_resident_and_staged_tiles_bitwise(N, tile, D):
    """Block-async under the persistent driver keeps each tile and a one-cell
    halo in LDS (three copies: a chunk's input survives it until the check
    that measured it is decided) and trades edges with its four neighbours
    after every chunk, where all tiles fit one round: 32 x 16 and 32 x 8 tiles
    at N = 256, ragged tiles one cell wide and high (N = 33), lone tiles
    (N = 1, 2), 64 x 60 tiles (four cells per thread, ragged 44 cells wide),
    one-column tiles.  Where one tile per block does not fit one round, each
    block holds a group of consecutive tiles (7 x 5 at N = 150, 32 x 16 at
    N = 1024: 2048 tiles, 32 x 8 at N = 700 and 16 x 16 at N = 1000, ragged,
    the last group short).  Tiles that no group fits in one round (64 x 64 at
    N = 1500: 576 tiles of 4096 cells) take re-staged tiles.  Both equal the
    oracle's block-async model bit for bit."""
    r = 10.0
    say("persist async tiles", N, tile, D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1])
    got = lib_solve(N, r, s, 3, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=tile[0], tile_y=tile[1], driver=PER))
    assert_same(got, ref, f"N={N} {tile} D={D}")


@pytest.mark.parametrize("N,D", [(200, 3), (200, 8), (1024, 8)])
def test_async_resident_nan_and_noconv(N, D):
    """A failed step ends the resident block-async solve with the oracle's
    status and field (the checked iterate, not the chunk run past it), with
    one tile per block (N = 200) and with two (N = 1024)."""
    r, tile = 10.0, (32, 16)
    say("persist async resident noconv/nan", N, D)
    s = workloads.gaussian_source(N, r)
    o = dict(kernel=jac.JAC_ASYNC, D=D, tile_x=tile[0], tile_y=tile[1], driver=PER)
    for cap in (8, 40, 41):
        ref = oracle.solve(N, r, s, steps=2, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1], max_sweeps=cap)
        assert ref.status == oracle.ENOCONV
        assert_same(lib_solve(N, r, s, 2, opts(max_sweeps=cap, **o)), ref, f"noconv D={D} cap={cap}")
    u0 = np.zeros((N, N), np.float32)
    u0[N // 3, N // 2] = np.inf
    ref = oracle.solve(N, r, s, u0=u0, steps=2, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1])
    assert ref.status == oracle.ENAN
    assert_same(lib_solve(N, r, s, 2, opts(**o), u0=u0), ref, f"nan D={D}")


@pytest.mark.parametrize("tile,D,r", [((32, 16), 8, 10.0), ((32, 8), 4, 10.0), ((32, 16), 8, 1.0)])
def test_config_c5_async_bitwise(tile, D, r):
    """N = 256, ten steps of block-async in one kernel with resident tiles."""
    say("persist C5 async", tile, D, r)
    s = workloads.gaussian_source(256, r)
    ref = oracle.solve(256, r, s, M=8, mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1])
    got = lib_solve(256, r, s, 10, opts(kernel=jac.JAC_ASYNC, D=D, tile_x=tile[0], tile_y=tile[1], driver=PER))
    assert_same(got, ref, f"C5 async {tile} D={D} r={r}")


@pytest.mark.parametrize("kernel,D", [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 8)])
@pytest.mark.parametrize("r", [1.0, 10.0])
def test_config_c5_bitwise(kernel, D, r):
    """N = 256, the launch-bound workload, ten steps in one kernel."""
    say("persist C5", kernel, D, r)
    s = workloads.gaussian_source(256, r)
    ref = oracle.solve(256, r, s)
    assert_same(lib_solve(256, r, s, 10, opts(kernel=kernel, D=D, driver=PER)), ref, f"C5 {kernel} r={r}")


@pytest.mark.parametrize("N,side", [(700, 0), (1024, 0), (300, 16), (33, 8), (300, 88), (300, 100), (1500, 0),
                                    (256, 0), (2, 0), (1, 0)])
def test_sync_resident_and_staged_tiles_bitwise(N, side):
    """The synchronous sweep under the persistent driver takes resident tiles
    (each block keeps its tile and a two-cell halo in LDS and trades edges with
    its neighbours after every sweep) where every tile fits one round --
    automatic 16-, 32- or 64-cell tiles up to N = 1024, 16-, 8- and 88-cell
    tiles, a lone 2 x 2 tile -- and re-staged tiles otherwise (100-cell tiles
    whose interior exceeds the block's cells, N = 1500, N = 1); both are the
    oracle's bits."""
    r = 10.0
    say("persist sync tiles", N, side)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3)
    assert_same(lib_solve(N, r, s, 3, opts(driver=PER, band_rows=side)), ref, f"N={N} side={side}")


def test_sync_resident_nan_and_noconv():
    """A failed step ends the resident solve with the oracle's status and field."""
    N, r = 200, 10.0
    say("persist sync resident noconv/nan")
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, max_sweeps=40)
    assert ref.status == oracle.ENOCONV
    assert_same(lib_solve(N, r, s, 2, opts(driver=PER, max_sweeps=40)), ref, "noconv")
    u0 = np.zeros((N, N), np.float32)
    u0[N // 3, N // 2] = np.inf
    ref = oracle.solve(N, r, s, u0=u0, steps=2)
    assert ref.status == oracle.ENAN
    assert_same(lib_solve(N, r, s, 2, opts(driver=PER), u0=u0), ref, "nan")


@pytest.mark.parametrize("N,side,D", [(101, 32, 4), (100, 32, 4), (256, 16, 15), (40, 8, 7), (256, 0, 8),
                                      (700, 0, 8), (1024, 0, 5), (1500, 0, 4), (257, 0, 16), (40, 8, 8)])
def test_tblock_resident_and_staged_tiles_bitwise(N, side, D):
    """Temporal blocking under the persistent driver keeps each tile and a
    halo H = D + 1 cells deep in LDS and takes the halo from its eight
    neighbours after every D sweeps where all tiles fit one round and every
    tile is at least H cells on a side: a ragged tile of exactly H (N = 101),
    tiles of side H (256, 16, 15 and 40, 8, 7), automatic 16-cell tiles
    (256), 64-cell tiles with an 82-cell region (700, 1024).  A ragged tile
    under H (N = 100, 257), a tile side under H (40, 8, 8) or more tiles than
    one round (1500) takes re-staged tiles.  Both are the oracle's bits."""
    r = 10.0
    say("persist tblock tiles", N, side, D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=max(8, D))
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=D, M=max(8, D), driver=PER, band_rows=side))
    assert_same(got, ref, f"N={N} side={side} D={D}")


@pytest.mark.parametrize("D", [3, 5, 8])
def test_tblock_resident_nan_and_noconv(D):
    """A failed step ends the resident temporal-blocking solve with the
    oracle's status and field, also where the sweep limit falls inside an
    interval of partial chunks (D = 3, 5 against an interval of 8)."""
    N, r = 200, 10.0
    say("persist tblock resident noconv/nan", D)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=8, max_sweeps=40)
    assert ref.status == oracle.ENOCONV
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=D, driver=PER, max_sweeps=40))
    assert_same(got, ref, f"noconv D={D}")
    u0 = np.zeros((N, N), np.float32)
    u0[N // 3, N // 2] = np.inf
    ref = oracle.solve(N, r, s, u0=u0, steps=2, M=8)
    assert ref.status == oracle.ENAN
    got = lib_solve(N, r, s, 2, opts(kernel=jac.JAC_TBLOCK, D=D, driver=PER), u0=u0)
    assert_same(got, ref, f"nan D={D}")


def test_config_c1_bitwise():
    say("persist C1")
    s = workloads.point_source(512, 1.0)
    ref = oracle.solve(512, 1.0, s)
    assert_same(lib_solve(512, 1.0, s, 10, opts(kernel=jac.JAC_TBLOCK, D=8, driver=PER)), ref, "C1")


def test_config_c2_against_stored_oracle():
    """N = 2048: more tiles than resident blocks, so blocks loop over tiles."""
    exp = load_expected("C2")
    say("persist C2")
    N, r = exp["N"], exp["r"]
    sol = jac.Solver(N, r, workloads.source(exp["source"], N, r))
    try:
        _, k, rho = sol.solve(exp["steps"], opts(kernel=jac.JAC_TBLOCK, D=8, driver=PER))
        assert k.tolist() == exp["sweeps"]
        assert [f"{v:08x}" for v in rho.view(np.uint32)] == exp["rho_bits"]
        assert field_hash(sol.field()) == exp["field_sha256"][-1]
    finally:
        sol.close()


def test_one_call_equals_step_by_step():
    N, r = 200, 10.0
    say("persist steps")
    s = workloads.gaussian_source(N, r)
    st, whole, k_whole, _ = lib_solve(N, r, s, 5, opts(kernel=jac.JAC_TBLOCK, D=4, driver=PER))
    sol = jac.Solver(N, r, s)
    try:
        ks = [sol.step(opts(kernel=jac.JAC_TBLOCK, D=4, driver=PER))[1] for _ in range(5)]
        assert ks == k_whole.tolist()
        assert np.array_equal(sol.field().view(np.uint32), whole.view(np.uint32))
    finally:
        sol.close()


def test_noconv_and_nan():
    N, r = 90, 100.0
    say("persist noconv")
    s = workloads.point_source(N, r)
    for cap in (1, 40, 41):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
        assert_same(lib_solve(N, r, s, 2, opts(driver=PER, max_sweeps=cap)), ref, f"cap {cap}")
    s2 = workloads.point_source(33, 1.0)
    s2[4, 4] = np.nan
    ref = oracle.solve(33, 1.0, s2, steps=2)
    st, u, k, rho = lib_solve(33, 1.0, s2, 2, opts(driver=PER))
    assert st == jac.JAC_ENAN and k.tolist() == ref.sweeps.tolist()
