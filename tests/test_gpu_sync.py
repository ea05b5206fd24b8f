"""Kernel (a), the synchronous sweep with its fused check, against the oracle bit
for bit: fields, per-step sweep counts and rho (page "stencil-jacobian.vercel.app",
section 02: every kernel reproduces the reference down to identical sweep
counts; grids such as N = 70 leave partial tiles to catch boundary bugs)."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, bits, field_hash, lib_solve, load_expected, opts, say

pytestmark = pytest.mark.gpu

SMALL_N = [1, 2, 3, 4, 5, 7, 8, 63, 64, 65, 70, 127, 129, 255, 256, 257, 300, 513]


@pytest.mark.parametrize("N", SMALL_N)
@pytest.mark.parametrize("kind,r", [("point", 1.0), ("gaussian", 10.0)])
def test_small_grids_bitwise(N, kind, r):
    say("sync small", N, kind, r)
    s = workloads.source(kind, N, r)
    ref = oracle.solve(N, r, s, steps=3)
    assert_same(lib_solve(N, r, s, 3, opts()), ref, f"N={N} {kind} r={r}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_fields_bitwise(seed):
    N, r = 97, 10.0
    say("sync random", seed)
    s = workloads.random_source(N, r, seed)
    u0 = workloads.random_field(N, seed)
    ref = oracle.solve(N, r, s, u0=u0, steps=2)
    assert_same(lib_solve(N, r, s, 2, opts(), u0=u0), ref, f"seed {seed}")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 16])
def test_check_interval_bitwise(M):
    """Odd intervals end a step in either buffer; counts stay multiples of M."""
    N, r = 70, 10.0
    say("sync M", M)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=3, M=M)
    assert_same(lib_solve(N, r, s, 3, opts(M=M)), ref, f"M={M}")


def test_config_c1_bitwise():
    """N = 512, r = 1, point source, ten steps (352 sweeps)."""
    c = workloads.CONFIGS["C1"]
    say("sync C1")
    s = workloads.source(c["source"], c["N"], c["r"])
    ref = oracle.solve(c["N"], c["r"], s)
    assert ref.total_sweeps == 352
    assert_same(lib_solve(c["N"], c["r"], s, 10, opts()), ref, "C1")


@pytest.mark.parametrize("r", [1.0, 10.0])
def test_config_c5_bitwise(r):
    """N = 256, Gaussian sigma = 16, ten steps."""
    say("sync C5", r)
    s = workloads.gaussian_source(256, r)
    ref = oracle.solve(256, r, s)
    assert_same(lib_solve(256, r, s, 10, opts()), ref, f"C5 r={r}")


def test_config_c2_bitwise():
    """N = 2048, r = 10, Gaussian, ten steps (2256 sweeps)."""
    say("sync C2")
    s = workloads.gaussian_source(2048, 10.0)
    ref = oracle.solve(2048, 10.0, s)
    assert ref.total_sweeps == 2256
    assert_same(lib_solve(2048, 10.0, s, 10, opts()), ref, "C2")


@pytest.mark.parametrize("name", ["C3"])
def test_large_config_against_stored_oracle_hashes(name):
    """N = 8192: the oracle's per-step sweeps, rho and field hashes were written by
    tests/golden/make_expected.py; every step must match bit for bit."""
    exp = load_expected(name)
    assert exp is not None, f"tests/golden/expected_{name}.json missing"
    say("sync golden", name)
    N, r = exp["N"], exp["r"]
    s = workloads.source(exp["source"], N, r)
    sol = jac.Solver(N, r, s)
    try:
        for n in range(exp["steps"]):
            st, k, rho = sol.step(opts(M=exp["M"]))
            assert k == exp["sweeps"][n], f"step {n}"
            assert f"{np.float32(rho).view(np.uint32):08x}" == exp["rho_bits"][n], f"step {n}"
            assert field_hash(sol.field()) == exp["field_sha256"][n], f"step {n}"
    finally:
        sol.close()


@pytest.mark.parametrize("checks", [jac.JAC_CHECKS_OVERLAPPED, jac.JAC_CHECKS_BLOCKING])
def test_long_band_form_on_ragged_grid_bitwise(checks):
    """N = 8190 gives 64-row wavefront bands on a 256-CU GPU (32 x 32
    workgroups: one balanced round), with a ragged last band and strip; two
    checked intervals, overlapped checks fused into the sweep or blocking ones
    by the residual-only kernel."""
    N, r = 8190, 10.0
    say("sync long bands", N, checks)
    s = workloads.gaussian_source(N, r)
    ref = oracle.solve(N, r, s, steps=1, M=8, max_sweeps=16)
    assert_same(lib_solve(N, r, s, 1, opts(max_sweeps=16, checks=checks)), ref, f"N={N} checks={checks}")


# ------------------------------------------------------------ driver edges

def test_max_sweeps_gives_noconv_and_keeps_checked_iterate():
    N, r = 64, 100.0
    say("sync noconv")
    s = workloads.point_source(N, r)
    for cap in (1, 8, 40, 41):
        ref = oracle.solve(N, r, s, steps=2, max_sweeps=cap)
        assert ref.status == oracle.ENOCONV
        assert_same(lib_solve(N, r, s, 2, opts(max_sweeps=cap)), ref, f"cap {cap}")


def test_nan_source_gives_enan():
    N, r = 33, 1.0
    say("sync nan")
    s = workloads.point_source(N, r)
    s[5, 6] = np.nan
    ref = oracle.solve(N, r, s, steps=2)
    assert ref.status == oracle.ENAN
    st, u, k, rho = lib_solve(N, r, s, 2, opts())
    assert st == jac.JAC_ENAN and k.tolist() == ref.sweeps.tolist() and np.isnan(rho[0])
    assert np.array_equal(np.isnan(u), np.isnan(ref.u))
    ok = ~np.isnan(u)
    assert np.array_equal(bits(u[ok]), bits(ref.u[ok]))


@pytest.mark.parametrize("kernel,D,tile", [(jac.JAC_SYNC, 1, (32, 8)), (jac.JAC_TBLOCK, 8, (32, 8)),
                                           (jac.JAC_TBLOCK, 11, (32, 8)), (jac.JAC_ASYNC, 8, (32, 16)),
                                           (jac.JAC_ASYNC, 4, (32, 8))])
def test_zero_problem_gives_enan(kernel, D, tile):
    """r = 0, s = 0 from u = 0: b_A = 0, the iterate stays 0 and the first
    check divides 0 by 0.  As in the oracle, the NaN rho ends the step with
    ENAN after 8 sweeps and leaves the zero field."""
    N = 300
    say("zero problem", kernel, D, tile)
    s = np.zeros((N, N), np.float32)
    kw = dict(mode=oracle.ASYNC, D=D, tx=tile[0], ty=tile[1]) if kernel == jac.JAC_ASYNC else {}
    ref = oracle.solve(N, 0.0, s, steps=2, **kw)
    assert ref.status == oracle.ENAN and ref.sweeps.tolist() == [8, 0]
    st, u, k, rho = lib_solve(N, 0.0, s, 2, opts(kernel=kernel, D=D, tile_x=tile[0], tile_y=tile[1]))
    assert st == jac.JAC_ENAN and k.tolist() == [8, 0] and np.isnan(rho[0]), (st, k, rho)
    assert not np.any(u)


@pytest.mark.parametrize("kernel,D,driver", [(jac.JAC_SYNC, 1, jac.JAC_LAUNCH), (jac.JAC_TBLOCK, 8, jac.JAC_LAUNCH),
                                             (jac.JAC_TBLOCK, 11, jac.JAC_LAUNCH), (jac.JAC_ASYNC, 8, jac.JAC_LAUNCH),
                                             (jac.JAC_SYNC, 1, jac.JAC_GRAPH), (jac.JAC_TBLOCK, 8, jac.JAC_PERSISTENT)])
def test_field_transfers_between_steps_bitwise(kernel, D, driver):
    """The host transfers stage the field in the idle iterate plane and then
    restore it: a field read after every step and written back after the
    second leave every step on the oracle's bits (ragged N = 301, random
    u^0 written in first)."""
    N, r = 301, 10.0
    say("field transfers", kernel, D, driver)
    s = workloads.gaussian_source(N, r)
    prev = workloads.random_field(N, 3)
    kw = dict(mode=oracle.ASYNC, D=D, tx=32, ty=16) if kernel == jac.JAC_ASYNC else {}
    o = opts(kernel=kernel, D=D, driver=driver, tile_x=32, tile_y=16 if kernel == jac.JAC_ASYNC else 8)
    sol = jac.Solver(N, r, s)
    try:
        sol.set_field(prev)
        for n in range(3):
            ref = oracle.solve(N, r, s, u0=prev, steps=1, **kw)
            st, k, rho = sol.step(o)
            u = sol.field()
            assert (st, k) == (jac.JAC_OK, int(ref.sweeps[0])), (n, st, k)
            assert np.float32(rho).view(np.uint32) == ref.rho[0].view(np.uint32), n
            assert np.array_equal(bits(u), bits(ref.u)), f"step {n}"
            if n == 1:
                sol.set_field(u)
            prev = ref.u
    finally:
        sol.close()


def test_zero_coupling_single_check():
    N = 40
    say("sync r=0")
    s = workloads.random_source(N, 1.0, 5) + np.float32(0.25)
    ref = oracle.solve(N, 0.0, s, steps=3)
    assert_same(lib_solve(N, 0.0, s, 3, opts()), ref, "r=0")


def test_fixed_sweeps_match_oracle():
    """jac_sweep: b from the field, then exactly n sweeps, and rho of the result."""
    N, r = 129, 10.0
    say("sync fixed sweeps")
    s = workloads.random_source(N, r, 9)
    u0 = workloads.random_field(N, 9)
    b = oracle.rhs(u0, s)
    sol = jac.Solver(N, r, s)
    try:
        want = u0
        for n in range(0, 6):
            sol.set_field(u0)
            rho = sol.sweep(n, opts(), want_rho=True)
            if n > 0:
                want = oracle.sweep(want, b, r)
            assert np.array_equal(bits(sol.field()), bits(want)), f"n={n}"
            R = oracle.residual(want, b, r)
            assert np.float32(rho) == np.float32(R) / oracle.rhs_norm(b, r)
    finally:
        sol.close()


def test_checkpoint_resume_is_bitwise():
    N, r = 150, 10.0
    say("sync checkpoint")
    s = workloads.gaussian_source(N, r)
    st, full, k_full, _ = lib_solve(N, r, s, 10, opts())
    a = jac.Solver(N, r, s)
    st1, k1, _ = a.solve(5, opts())
    mid = a.field()
    a.close()
    b = jac.Solver(N, r, s)
    b.set_field(mid)
    st2, k2, _ = b.solve(5, opts())
    end = b.field()
    b.close()
    assert k_full.tolist() == k1.tolist() + k2.tolist()
    assert np.array_equal(bits(full), bits(end))


def test_repeat_and_reset_are_deterministic():
    N, r = 200, 10.0
    say("sync determinism")
    s = workloads.gaussian_source(N, r)
    sol = jac.Solver(N, r, s)
    try:
        _, k1, r1 = sol.solve(4, opts())
        u1 = sol.field()
        sol.reset()
        assert not sol.field().any()
        _, k2, r2 = sol.solve(4, opts())
        u2 = sol.field()
    finally:
        sol.close()
    assert k1.tolist() == k2.tolist() and np.array_equal(bits(r1), bits(r2))
    assert np.array_equal(bits(u1), bits(u2))


def test_profile_counts_launches(monkeypatch):
    monkeypatch.setenv("JACOBI_PREDICT_MARGIN", "0")  # every check fused, as counted below
    N, r = 256, 1.0
    say("sync profile")
    s = workloads.gaussian_source(N, r)
    sol = jac.Solver(N, r, s)
    try:
        sol.profile(1)
        _, k, _ = sol.solve(2, opts())
        ms, n, nt = sol.profile_read("sync")
        ms_c, n_c, _ = sol.profile_read("sync_check")
        _, n_r, _ = sol.profile_read("rhs")
        _, n_noop, _ = sol.profile_read("noop")
        _, n_red, _ = sol.profile_read("reduce")
    finally:
        sol.close()
    assert n_r == 2 and nt == n
    checks = int(k.sum()) // 8
    # each step: group 0 has 8 plain sweeps, groups 1..g-1 one checking + 7 plain,
    # the stopping check runs, and what was queued after it returns at once
    assert n_c == checks
    assert n == 8 * 2 + 7 * (checks - 2)
    assert n_noop == 2 * (7 + 8)
    assert n_red == 2 + checks + 2  # two norms, every check, the no-op groups' reductions
    assert ms > 0 and ms_c > 0
