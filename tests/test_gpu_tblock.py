"""Kernel (b), exact temporal blocking, against the oracle bit for bit (page
"stencil-jacobian.vercel.app", section 02: after D sweeps the tile holds exactly
what D synchronous sweeps would produce).  A launch does up to D sweeps; checks
fall every M = 8 sweeps whatever D (a launch deeper than 8 measures the residual
at the levels where checks fall), so every depth gives the oracle's sweep
counts at M = 8; with M = D the interval is D."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, bits, field_hash, lib_solve, load_expected, opts, say

pytestmark = pytest.mark.gpu

TB = jac.JAC_TBLOCK


def interval(D, M=8):
    return M


@pytest.mark.parametrize("D", list(range(1, 17)))
@pytest.mark.parametrize("N", [70, 300])
def test_every_depth_bitwise(D, N):
    r = 10.0
    say("tblock depth", D, N)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=interval(D))
    assert_same(lib_solve(N, r, s, 2, opts(kernel=TB, D=D)), ref, f"D={D} N={N}")


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 9, 15, 63, 64, 65, 127, 129, 224, 240, 248, 249, 255, 256,
                               257, 260, 264, 481, 496, 500, 504, 508, 512, 513, 740, 744, 1000])
@pytest.mark.parametrize("D", [2, 4, 8])
def test_small_and_ragged_grids_bitwise(N, D):
    """Window widths 248/240 (D 2-4 / 8) and band heights meet N at every offset;
    N a multiple of 4 from 256 on takes the aligned strip layout (first window
    at column 0, last window ending at column N-1), the others the general one."""
    r = 1.0
    say("tblock small", N, D)
    s = workloads.point_source(N, r)
    ref = oracle.solve(N, r, s, steps=2, M=interval(D))
    assert_same(lib_solve(N, r, s, 2, opts(kernel=TB, D=D)), ref, f"N={N} D={D}")


@pytest.mark.parametrize("D", [3, 5, 12])
def test_random_fields_bitwise(D):
    N, r = 181, 100.0
    say("tblock random", D)
    s = workloads.random_source(N, r, D)
    u0 = workloads.random_field(N, D)
    ref = oracle.solve(N, r, s, u0=u0, steps=1, M=interval(D))
    assert_same(lib_solve(N, r, s, 1, opts(kernel=TB, D=D), u0=u0), ref, f"D={D}")


@pytest.mark.parametrize("D", [2, 4, 8, 11])
def test_config_c1_bitwise(D):
    say("tblock C1", D)
    s = workloads.point_source(512, 1.0)
    ref = oracle.solve(512, 1.0, s)
    assert_same(lib_solve(512, 1.0, s, 10, opts(kernel=TB, D=D)), ref, f"C1 D={D}")


@pytest.mark.parametrize("D", [4, 8])
@pytest.mark.parametrize("r", [1.0, 10.0])
def test_config_c5_bitwise(D, r):
    say("tblock C5", D, r)
    s = workloads.gaussian_source(256, r)
    ref = oracle.solve(256, r, s)
    assert_same(lib_solve(256, r, s, 10, opts(kernel=TB, D=D)), ref, f"C5 D={D} r={r}")


@pytest.mark.parametrize("D", [2, 4, 8])
def test_config_c2_against_stored_oracle(D):
    """N = 2048, r = 10: D in {2, 4, 8} with M = 8 keeps the oracle's counts."""
    exp = load_expected("C2")
    assert exp is not None
    say("tblock C2", D)
    N, r = exp["N"], exp["r"]
    sol = jac.Solver(N, r, workloads.source(exp["source"], N, r))
    try:
        for n in range(exp["steps"]):
            _, k, rho = sol.step(opts(kernel=TB, D=D))
            assert k == exp["sweeps"][n]
            assert f"{np.float32(rho).view(np.uint32):08x}" == exp["rho_bits"][n]
            assert field_hash(sol.field()) == exp["field_sha256"][n], f"step {n}"
    finally:
        sol.close()


@pytest.mark.parametrize("D", [4, 8])
def test_config_c3_against_stored_oracle(D):
    """N = 8192, r = 10, the benchmark workload: step by step, then all ten steps
    in one solve call with the default options, as the benchmark times it."""
    exp = load_expected("C3")
    assert exp is not None
    say("tblock C3", D)
    N, r = exp["N"], exp["r"]
    sol = jac.Solver(N, r, workloads.source(exp["source"], N, r))
    try:
        for n in range(exp["steps"]):
            _, k, rho = sol.step(opts(kernel=TB, D=D))
            assert k == exp["sweeps"][n]
            assert f"{np.float32(rho).view(np.uint32):08x}" == exp["rho_bits"][n]
            assert field_hash(sol.field()) == exp["field_sha256"][n], f"step {n}"
        sol.reset()
        st, k, rho = sol.solve(exp["steps"], jac.jac_opts_default(kernel=TB, D=D))
        assert st == jac.JAC_OK and k.tolist() == exp["sweeps"]
        assert [f"{np.float32(x).view(np.uint32):08x}" for x in rho] == exp["rho_bits"]
        assert field_hash(sol.field()) == exp["field_sha256"][-1]
    finally:
        sol.close()


def test_fixed_sweep_counts_not_multiple_of_D():
    """jac_sweep with n = qD + p: q launches of D and one of p sweeps."""
    N, r = 143, 10.0
    say("tblock fixed sweeps")
    s = workloads.random_source(N, r, 4)
    u0 = workloads.random_field(N, 4)
    b = oracle.rhs(u0, s)
    sol = jac.Solver(N, r, s)
    try:
        for n in (1, 5, 8, 13):
            sol.set_field(u0)
            rho = sol.sweep(n, opts(kernel=TB, D=5), want_rho=True)
            want = u0
            for _ in range(n):
                want = oracle.sweep(want, b, r)
            assert np.array_equal(bits(sol.field()), bits(want)), f"n={n}"
            assert np.float32(rho) == oracle.residual(want, b, r) / oracle.rhs_norm(b, r)
    finally:
        sol.close()


def test_noconv_keeps_checked_iterate():
    N, r = 90, 100.0
    say("tblock noconv")
    s = workloads.point_source(N, r)
    for cap, D in ((20, 4), (16, 16), (64, 8)):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap, M=interval(D))
        assert ref.status == oracle.ENOCONV
        assert_same(lib_solve(N, r, s, 2, opts(kernel=TB, D=D, max_sweeps=cap)), ref, f"cap {cap} D {D}")


def test_d_out_of_range_rejected():
    sol = jac.Solver(16, 1.0)
    try:
        for D in (0, 17):
            st, _, _ = jac.jac_step(sol.ctx, opts(kernel=TB, D=D))
            assert st == jac.JAC_EINVAL
    finally:
        sol.close()


@pytest.mark.parametrize("H", [1, 2, 3, 7, 33, 1000])
def test_band_heights_bitwise(H):
    """Any band height (rows per wavefront) gives the same bits."""
    N, r, D = 150, 10.0, 6
    say("tblock band", H)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=2)
    assert_same(lib_solve(N, r, s, 2, opts(kernel=TB, D=D, band_rows=H)), ref, f"H={H}")


_ALIGNED_REF = {}


@pytest.mark.parametrize("H", [4, 64, 0, 1040])
@pytest.mark.parametrize("D", [5, 7, 8, 9, 12, 16])
def test_aligned_layout_tall_bands_bitwise(D, H):
    """The aligned strip layout (N a multiple of 4, N >= 256: windows inside the
    grid, no column masking) with short, automatic and full-height bands, both
    stream directions, buffer row I/O and the straight (all levels exact) row
    path, against the oracle on a grid whose bands are taller than the
    pipeline (N = 1040)."""
    N, r = 1040, 10.0
    say("tblock aligned", D, H)
    s = workloads.gaussian_source(N, r)
    M = interval(D)
    if M not in _ALIGNED_REF:
        _ALIGNED_REF[M] = oracle.solve(N, r, s, steps=2, M=M)
    assert_same(lib_solve(N, r, s, 2, opts(kernel=TB, D=D, M=8, band_rows=H)), _ALIGNED_REF[M], f"D={D} H={H}")


def _c3_against(exp, o):
    N, r = exp["N"], exp["r"]
    sol = jac.Solver(N, r, workloads.source(exp["source"], N, r))
    try:
        st, k, rho = sol.solve(exp["steps"], o)
        assert st == jac.JAC_OK and k.tolist() == exp["sweeps"], (k.tolist(), exp["sweeps"])
        assert [f"{np.float32(x).view(np.uint32):08x}" for x in rho] == exp["rho_bits"]
        assert field_hash(sol.field()) == exp["field_sha256"][-1]
    finally:
        sol.close()


@pytest.mark.parametrize("D", list(range(1, 17)))
def test_config_c3_every_depth_against_stored_oracle(D):
    """N = 8192, r = 10, the benchmark workload, at every depth 1..16 in one
    ten-step solve with the default options (checks every 8 sweeps; from D = 9
    on deep launches check inner levels): per-step sweeps and rho bits and the
    final field against the oracle's."""
    exp = load_expected("C3")
    assert exp is not None and exp["M"] == 8
    say("tblock C3 depth", D)
    _c3_against(exp, jac.jac_opts_default(kernel=TB, D=D))


@pytest.mark.parametrize("D", list(range(9, 17)))
def test_config_c3_interval_d_against_stored_oracle(D):
    """The same workload checked every D sweeps (M = D): launches of D sweeps
    that check their input, against the oracle run with M = D."""
    exp = load_expected(f"C3_M{D}")
    assert exp is not None and exp["M"] == D
    say("tblock C3 interval D", D)
    _c3_against(exp, jac.jac_opts_default(kernel=TB, D=D, M=D))


@pytest.mark.parametrize("N,D,r", [(70, 8, 10.0), (300, 4, 0.05), (513, 3, 1.0), (1040, 8, 10.0)])
def test_first_launch_forms_rhs_bitwise(N, D, r):
    """Overlapped checks through the launch driver: each step's first launch
    forms b = u^n + s itself and leaves the partial maxima of |b_A|, and no
    separate right-hand-side pass runs; blocking checks and the graph driver
    keep the separate pass.  Every path gives the oracle's bits (random u^0, so
    b differs from s; at r = 0.05 the interior, not row 0, sets ||b_A||)."""
    say("tblock rhs in first launch", N, D, r)
    s = workloads.random_source(N, r, 11)
    u0 = workloads.random_field(N, 11)
    ref = oracle.solve(N, r, s, u0=u0, steps=3)
    for checks, driver, fused in ((jac.JAC_CHECKS_OVERLAPPED, jac.JAC_LAUNCH, True),
                                  (jac.JAC_CHECKS_BLOCKING, jac.JAC_LAUNCH, False),
                                  (jac.JAC_CHECKS_OVERLAPPED, jac.JAC_GRAPH, False)):
        sol = jac.Solver(N, r, s)
        try:
            sol.set_field(u0)
            sol.profile(1)
            st, k, rho = sol.solve(3, opts(kernel=TB, D=D, checks=checks, driver=driver))
            u = sol.field()
            _, n_rhs, _ = sol.profile_read("rhs")
            _, n_first, _ = sol.profile_read("tblock_rhs")
            fast = sol.last_division_fast
        finally:
            sol.close()
        assert_same((st, u, k, rho), ref, f"N={N} D={D} checks={checks} driver={driver}")
        # the forming launch exists for the constant-divisor quotient only
        assert fast or r < 1.0
        assert (n_rhs, n_first) == ((0, 3) if fused and fast else (3, 0)), (checks, driver, fast)


def test_band_spanning_more_than_2gib_bitwise():
    """N = 24576 asked for as one band of rows at D = 8: its rows span 2.4 GB,
    past the 32-bit offsets of the buffer row I/O, so the library lowers the
    band height.  After the step's first launch (which also forms b), every
    point must equal the oracle's value for a point at the same distance from
    the ghost ring on a 40 x 40 grid with the same constant source: from u = 0,
    8 sweeps see only 8 cells around a point, and the rest is translation
    invariant."""
    N, r, D, c, n = 24576, 1.0, 8, np.float32(0.25), 40
    say("tblock band over 2 GiB", N, D)
    ref = oracle.solve(n, r, np.full((n, n), c, np.float32), steps=1, max_sweeps=8)
    assert ref.status == oracle.ENOCONV and ref.sweeps[0] == 8
    sol = jac.Solver(N, r, np.full((N, N), c, np.float32))
    try:
        st, k, rho = sol.step(opts(kernel=TB, D=D, band_rows=N, max_sweeps=8), allow=(jac.JAC_ENOCONV,))
        u = sol.field()
    finally:
        sol.close()
    assert st == jac.JAC_ENOCONV and k == 8
    assert np.float32(rho).view(np.uint32) == ref.rho[0].view(np.uint32)
    idx = np.full(N, n // 2)
    idx[: n // 2] = np.arange(n // 2)
    idx[N - n // 2:] = np.arange(n // 2, n)
    for r0 in range(0, N, 4096):  # row blocks keep the expected array small
        want = ref.u[idx[r0:r0 + 4096, None], idx[None, :]]
        got = u[r0:r0 + 4096]
        assert np.array_equal(bits(got), bits(want)), f"rows {r0}..{r0 + 4095}"


@pytest.mark.parametrize("kernel,D", [(TB, 8), (TB, 11), (jac.JAC_SYNC, 1)])
def test_config_c4_against_stored_oracle(kernel, D):
    """N = 18432, r = 100, point source, ten steps (14160 sweeps), every step
    against the oracle's stored field hash (D = 11: launches of 11 sweeps over
    checks every 8, the fastest form at this size)."""
    exp = load_expected("C4")
    assert exp is not None
    say("C4", kernel, D)
    N, r = exp["N"], exp["r"]
    sol = jac.Solver(N, r, workloads.source(exp["source"], N, r))
    try:
        for n in range(exp["steps"]):
            _, k, rho = sol.step(opts(kernel=kernel, D=D))
            assert k == exp["sweeps"][n], f"step {n}"
            assert f"{np.float32(rho).view(np.uint32):08x}" == exp["rho_bits"][n]
            assert field_hash(sol.field()) == exp["field_sha256"][n], f"step {n}"
    finally:
        sol.close()


@pytest.mark.parametrize("D", [8, 5, 4, 1])
def test_sampled_checks_bitwise(D, monkeypatch):
    """Launches of at most 8 sweeps measure the residual of their input; a
    check not expected to stop takes it on every 8th row (a lower bound of R
    that decides a going-on check exactly), and a sample below tol is measured
    again in full, the step then stopping or going on with the interval after
    the check.  Row 0 alone (stride 2^20) forces many such second
    measurements; stride 0 turns sampling off.  All give the oracle's bits."""
    N, r = 300, 10.0
    s = workloads.gaussian_source(N, r)
    u0 = workloads.random_field(N, 7)
    ref = oracle.solve(N, r, s, u0=u0, steps=3, M=8)
    counts = {}
    for stride in ("0", "8", "1048576"):
        monkeypatch.setenv("JACOBI_SAMPLED_CHECKS", stride)
        say("tblock sampled", D, stride)
        sol = jac.Solver(N, r, s)
        try:
            sol.set_field(u0)
            sol.profile(1)
            st, k, rho = sol.solve(3, opts(kernel=jac.JAC_TBLOCK, D=D))
            got = (st, sol.field(), k, rho)
            counts[stride] = sol.profile_read("residual")[1]
        finally:
            sol.close()
        assert_same(got, ref, f"D={D} stride={stride}")
    assert counts["1048576"] > counts["0"]
