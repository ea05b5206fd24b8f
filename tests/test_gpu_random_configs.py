"""Seeded random combinations of the options, each against the oracle bit for
bit: ragged and tiny grids, couplings from 0.05 to 100, every kernel and
driver, blocking and overlapped checks, check intervals 1..12, depths up to
16 (temporal blocking) and 32 (block-async), odd tile shapes, sweep caps and
random initial fields; a second group on grids of 511 to 1100.  The
combinations are fixed by the seeds, so a failure
names a case that repeats (page "stencil-jacobian.vercel.app", sections 01
and 02: the step, the check every M sweeps, the three kernels)."""
import numpy as np
import pytest

import jacobi_stencil_amd as jac
import oracle
import workloads
from tests.gpu_helpers import assert_same, bits, opts, say

pytestmark = pytest.mark.gpu

KERNELS = {"sync": jac.JAC_SYNC, "tblock": jac.JAC_TBLOCK, "async": jac.JAC_ASYNC, "unfused": jac.JAC_SYNC_UNFUSED}
DRIVERS = {"launch": jac.JAC_LAUNCH, "graph": jac.JAC_GRAPH, "persistent": jac.JAC_PERSISTENT}
CHECKS = {"overlapped": jac.JAC_CHECKS_OVERLAPPED, "blocking": jac.JAC_CHECKS_BLOCKING}


def make_cases(n=48, seed=20261202, first=0, large=False):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(first, first + n):
        kernel = str(rng.choice(list(KERNELS)))
        driver = str(rng.choice(list(DRIVERS)))
        if kernel == "unfused" and driver == "persistent":
            driver = "launch"
        sizes = [1, 2, 3, 5, 17, 33, 64, 70, 97, 128, 150, 255, 256, 257, 300, 384, 400]
        if large:
            sizes = [511, 512, 513, 640, 777, 1024, 1100]
        if driver == "persistent":
            sizes = [s for s in sizes if s <= 300] or [512, 513, 1024]
        N = int(rng.choice(sizes))
        couplings = [0.05, 1.0, 10.0] if large else [0.05, 1.0, 10.0, 100.0]
        c = {"i": i, "N": N, "r": float(rng.choice(couplings)), "kernel": kernel,
             "driver": driver, "checks": str(rng.choice(list(CHECKS))), "M": int(rng.integers(1, 13)),
             "D": 1, "tile": (32, 8), "cap": 10**6, "u0": bool(rng.integers(0, 2)),
             "source": str(rng.choice(["gaussian", "random", "point"]))}
        if kernel == "tblock":
            c["D"] = int(rng.integers(1, 17))
        elif kernel == "async":
            c["D"] = int(rng.integers(1, 33))
            while True:
                tx = int(rng.choice([1, 3, 4, 7, 8, 16, 24, 32, 64]))
                ty = int(rng.choice([1, 2, 4, 8, 13, 16, 32]))
                if tx * ty <= 4096 and (driver != "persistent" or tx * ty >= 16):
                    break
            c["tile"] = (tx, ty)
        if rng.integers(0, 4) == 0:
            c["cap"] = int(rng.integers(1, 60))
        cases.append(c)
    return cases


CASES = make_cases() + make_cases(n=48, seed=7, first=48, large=True)


def source(c):
    N, r = c["N"], c["r"]
    if c["source"] == "gaussian":
        return workloads.gaussian_source(N, r)
    if c["source"] == "point":
        return workloads.point_source(N, r)
    return workloads.random_source(N, r, 100 + c["i"])


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['i']}" for c in CASES])
def test_random_configuration_bitwise(c):
    say("random config", c)
    N, r = c["N"], c["r"]
    s = source(c)
    u0 = workloads.random_field(N, 200 + c["i"]) if c["u0"] else None
    if c["kernel"] == "async":
        ref = oracle.solve(N, r, s, u0=u0, steps=2, M=c["M"], mode=oracle.ASYNC, D=c["D"], tx=c["tile"][0],
                           ty=c["tile"][1], max_sweeps=c["cap"])
    else:
        ref = oracle.solve(N, r, s, u0=u0, steps=2, M=c["M"], max_sweeps=c["cap"])
    o = opts(kernel=KERNELS[c["kernel"]], driver=DRIVERS[c["driver"]], D=c["D"], tile_x=c["tile"][0],
             tile_y=c["tile"][1], M=c["M"], max_sweeps=c["cap"], checks=CHECKS[c["checks"]])
    sol = jac.Solver(N, r, s)
    try:
        if u0 is not None:
            sol.set_field(u0)
        try:
            st, k, rho = sol.solve(2, o, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN))
        except jac.JacobiError as e:
            # block-async tiles under 64 points can need more check slots than
            # the workspace holds: rejected before any work runs
            assert c["kernel"] == "async" and c["tile"][0] * c["tile"][1] < 64, str(e)
            assert "tile too small" in str(e)
            want = u0 if u0 is not None else np.zeros((N, N), np.float32)
            assert np.array_equal(sol.field(), want)
            return
        res = (st, sol.field(), k, rho)
    finally:
        sol.close()
    assert_same(res, ref, str(c))


def make_sweep_cases(n=32, seed=5):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kernel = str(rng.choice(list(KERNELS)))
        c = {"i": i, "N": int(rng.choice([1, 2, 9, 64, 97, 130, 256, 301, 513])),
             "r": float(rng.choice([0.05, 1.0, 10.0, 100.0])), "kernel": kernel, "D": 1, "tile": (32, 8),
             "n": int(rng.integers(0, 41))}
        if kernel == "tblock":
            c["D"] = int(rng.integers(1, 17))
        elif kernel == "async":
            c["D"] = int(rng.integers(1, 33))
            tx = int(rng.choice([1, 3, 4, 8, 16, 24, 32, 64]))
            ty = int(rng.choice([1, 2, 4, 8, 13, 16, 32]))
            c["tile"] = (tx, ty)
        cases.append(c)
    return cases


SWEEP_CASES = make_sweep_cases()


@pytest.mark.parametrize("c", SWEEP_CASES, ids=[f"sweeps{c['i']}" for c in SWEEP_CASES])
def test_random_fixed_sweeps_bitwise(c):
    """jac_sweep and jac_sweep_static from the same random field: b = u^n + s,
    then exactly n sweeps -- for temporal blocking and block-async q launches
    of D and one of the remaining n - qD -- and rho of the result, against the
    oracle's single sweep and single block-asynchronous launch composed."""
    say("random fixed sweeps", c)
    N, r, n, D = c["N"], c["r"], c["n"], c["D"]
    s = workloads.random_source(N, r, 300 + c["i"])
    u0 = workloads.random_field(N, 400 + c["i"])
    b = oracle.rhs(u0, s)
    want = u0
    if c["kernel"] == "async":
        tx, ty = c["tile"]
        for q in range(0, n, D):
            want = oracle.async_launch(want, b, r, tx, ty, min(D, n - q))
    else:
        for _ in range(n):
            want = oracle.sweep(want, b, r)
    want_rho = np.float32(oracle.residual(want, b, r)) / oracle.rhs_norm(b, r)
    o = opts(kernel=KERNELS[c["kernel"]], D=D, tile_x=c["tile"][0], tile_y=c["tile"][1])
    sol = jac.Solver(N, r, s)
    try:
        for fn in (jac.jac_sweep, jac.jac_sweep_static):
            sol.set_field(u0)
            st, rho = fn(sol.ctx, o, n, True)
            assert st == jac.JAC_OK, jac.jac_last_error()
            assert np.array_equal(bits(sol.field()), bits(want)), f"{fn.__name__} {c}"
            assert np.float32(rho).view(np.uint32) == np.float32(want_rho).view(np.uint32), (fn.__name__, rho,
                                                                                            want_rho)
    finally:
        sol.close()


def make_study_cases(n=32, seed=9):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        tx = int(rng.choice([1, 3, 4, 8, 16, 24, 32, 64]))
        ty = int(rng.choice([1, 2, 4, 8, 13, 16, 32]))
        o = int(rng.integers(0, 9))
        while (tx + 2 * o) * (ty + 2 * o) > 4096:
            o -= 1
        ctrl = str(rng.choice(["static", "asc", "desc"]))
        c = {"i": i, "N": int(rng.choice([17, 64, 97, 150, 256, 300])), "r": float(rng.choice([1.0, 10.0, 100.0])),
             "D": int(rng.integers(1, 17)), "tile": (tx, ty), "o": o, "ctrl": ctrl, "M": int(rng.integers(1, 13)),
             "checks": "blocking" if ctrl != "static" else str(rng.choice(list(CHECKS))),
             "driver": "launch" if ctrl != "static" else str(rng.choice(["launch", "graph"]))}
        cases.append(c)
    return cases


STUDY_CASES = make_study_cases()
CTRL = {"static": (jac.JAC_STATIC, oracle.STATIC), "asc": (jac.JAC_G_ASC, oracle.G_ASC),
        "desc": (jac.JAC_G_DESC, oracle.G_DESC)}


@pytest.mark.parametrize("c", STUDY_CASES, ids=[f"study{c['i']}" for c in STUDY_CASES])
def test_random_overlap_and_controllers_bitwise(c):
    """Block-async with overlapping tiles (o cells per side, the page
    "Hierarchical Jacobi Iteration ...", section 3.5) and the G-asc / G-desc
    depth controllers (page "stencil-jacobian.vercel.app", section 02) on
    random tilings, depths, intervals and grids, against the oracle."""
    say("random overlap / controller", c)
    N, r = c["N"], c["r"]
    s = workloads.random_source(N, r, 500 + c["i"])
    lib_ctrl, orc_ctrl = CTRL[c["ctrl"]]
    tx, ty = c["tile"]
    ref = oracle.solve(N, r, s, steps=2, M=c["M"], mode=oracle.ASYNC, D=c["D"], tx=tx, ty=ty, o=c["o"],
                       controller=orc_ctrl)
    o = opts(kernel=jac.JAC_ASYNC, D=c["D"], tile_x=tx, tile_y=ty, M=c["M"], overlap=c["o"], controller=lib_ctrl,
             checks=CHECKS[c["checks"]], driver=DRIVERS[c["driver"]])
    sol = jac.Solver(N, r, s)
    try:
        st, k, rho = sol.solve(2, o, allow=(jac.JAC_ENOCONV, jac.JAC_ENAN))
        res = (st, sol.field(), k, rho)
    finally:
        sol.close()
    assert_same(res, ref, str(c))
