"""Measurement studies around the solver, on one GPU (results as JSON lines).

    python -m jacobi_stencil_amd.study checks      [--out FILE]
    python -m jacobi_stencil_amd.study regimes     [--out FILE] [--quick]
    python -m jacobi_stencil_amd.study controllers [--out FILE]
    python -m jacobi_stencil_amd.study overlap     [--out FILE]
    python -m jacobi_stencil_amd.study depths      [--out FILE]
    python -m jacobi_stencil_amd.study launches    [--out FILE]
    python -m jacobi_stencil_amd.study fit REGIMES_JSONL

What each one measures (page "stencil-jacobian.vercel.app" unless noted):

checks       time-to-solution against the check interval M, with blocking and
             overlapped checks (section 04, Table V; section 07: the host round
             trip of the convergence check is the synchronization that costs).
regimes      the c * s decomposition across grid sizes (section 05): for every
             strategy x, s = sweeps_x / sweeps_sync and
             c = (T_x / sweeps_x) / (T_sync / sweeps_sync), so the speed-up
             over the fused synchronous sweep is 1 / (c * s); also the unfused
             synchronous sweep (Table VI) and the time per sweep.
controllers  the depth controllers G-asc, G-desc and G-fb against static depths
             for the block-asynchronous kernel (section 06).
overlap      overlapping subdomains for the block-asynchronous kernel (Islam &
             Wang, "Hierarchical Jacobi Iteration ...", sections 3.5 and 4):
             sweeps and time against the overlap o.
depths       the depth sweep D = 1..16 at N = 8192, r = 10 for exact temporal
             blocking and for block-async at 32 x 16 tiles (section 05, Fig. 6 /
             Table VIII): time to solution, sweeps, s and c (checks every 8
             sweeps, every D above 8), and for launches of D sweeps (timed in a
             solve that checks every D sweeps) their mean device time, the HBM
             fraction of 12 bytes per point moved once per launch (8 TB/s) and
             the VALU fraction of 8 lane-operations per point-update (39.3 T/s).
launches     the cost of one launch in the launch-bound regime (section 04:
             about 4.4 us per synchronous sweep, 9.4 us for BA_D1, 19.4 us for
             BA_D8): at N = 256 and 512, r = 10, the mean device time of each
             launch class (HIP events around every launch) and the wall time per
             launch of a whole solve (solve time / launches), per kernel and
             driver, median of the repeats.
fit          a depth-2 decision tree on (working set / cache, r) picking the
             fastest family of the regimes study, with leave-one-size-out
             accuracy (section 06, "Depth-2 decision tree").

Timing: the whole solve (every step, check and host decision) between two
device synchronizations, median of `--repeats` after one warm-up solve, inputs
resident on the device.  Sources follow the workloads of the benchmark
(Gaussian, sigma = N/16).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X caches: 4 MiB L2 per XCD (8 XCDs), 256 MiB Infinity Cache (MALL).
L2_BYTES = 8 * 4 * 2**20
MALL_BYTES = 256 * 2**20


def _emit(out, rec):
    line = json.dumps(rec)
    print(line, flush=True)
    if out:
        with open(out, "a") as f:
            f.write(line + "\n")


class Runner:
    def __init__(self, repeats):
        import torch

        import jacobi_stencil_amd as jac
        import workloads

        self.torch, self.jac, self.wl = torch, jac, workloads
        self.repeats = repeats
        torch.cuda.set_device(0)
        self.sol = None
        self.key = None

    def solver(self, N, r):
        if self.key != (N, r):
            if self.sol is not None:
                self.sol.close()
                self.sol = None
                self.torch.cuda.empty_cache()
            self.sol = self.jac.Solver(N, r, self.wl.gaussian_source(N, r))
            self.key = (N, r)
        return self.sol

    def run(self, N, r, steps, **o):
        """Median time (ms) of a full solve, its sweeps and depth changes."""
        sol = self.solver(N, r)
        opts = self.jac.jac_opts_default(**o)
        sync = self.torch.cuda.synchronize
        sol.reset()
        sol.solve(steps, opts)
        sync()
        ts = []
        k = None
        for _ in range(self.repeats):
            sol.reset()
            sync()
            t0 = time.perf_counter()
            _, k, rho = sol.solve(steps, opts)
            sync()
            ts.append((time.perf_counter() - t0) * 1e3)
        dl = sol.depth_log()
        changes = int(sum(1 for i in range(1, len(dl)) if dl[i] != dl[i - 1]))
        sweeps = int(k.sum())
        ms = statistics.median(ts)
        return dict(N=N, r=r, steps=steps, ms=round(ms, 3), sweeps=sweeps,
                    gpts=round(N * N * sweeps / (ms / 1e3) / 1e9, 2), us_per_sweep=round(ms * 1e3 / sweeps, 3),
                    depth_changes=changes, rho_max=float(max(rho)))


def study_checks(a):
    R = Runner(a.repeats)
    jac = R.jac
    for N, kernel, D, driver in ((256, jac.JAC_SYNC, 1, jac.JAC_LAUNCH), (256, jac.JAC_SYNC, 1, jac.JAC_GRAPH),
                                 (256, jac.JAC_TBLOCK, 8, jac.JAC_LAUNCH), (8192, jac.JAC_SYNC, 1, jac.JAC_LAUNCH),
                                 (8192, jac.JAC_TBLOCK, 8, jac.JAC_LAUNCH)):
        for M in (1, 2, 4, 8, 16, 32):
            if kernel == jac.JAC_TBLOCK and M < D:
                continue
            for checks in (jac.JAC_CHECKS_BLOCKING, jac.JAC_CHECKS_OVERLAPPED):
                rec = R.run(N, 10.0, 10, kernel=kernel, D=D, M=M, driver=driver, checks=checks)
                rec.update(study="checks", kernel=kernel, D=D, M=M, driver=driver,
                           checks="blocking" if checks else "overlapped")
                _emit(a.out, rec)


def study_regimes(a):
    R = Runner(a.repeats)
    jac = R.jac
    sizes = (256, 1024, 4096, 8192) if a.quick else (256, 512, 1024, 2048, 4096, 8192, 16384, 18432)
    families = [("sync", dict(kernel=jac.JAC_SYNC)),
                ("sync_unfused", dict(kernel=jac.JAC_SYNC_UNFUSED)),
                ("temporal_D4", dict(kernel=jac.JAC_TBLOCK, D=4)),
                ("temporal_D8", dict(kernel=jac.JAC_TBLOCK, D=8)),
                ("async_D4_32x8", dict(kernel=jac.JAC_ASYNC, D=4, tile_x=32, tile_y=8)),
                ("async_D8_32x16", dict(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=16))]
    for N in sizes:
        rs = (1.0, 10.0, 100.0) if N <= 4096 else (1.0, 10.0)
        steps = 10 if N <= 8192 else 2
        for r in rs:
            base = None
            for name, o in families:
                rec = R.run(N, r, steps, **o)
                if base is None:
                    base = rec
                s = rec["sweeps"] / base["sweeps"]
                c = (rec["ms"] / rec["sweeps"]) / (base["ms"] / base["sweeps"])
                rec.update(study="regimes", family=name, s=round(s, 4), c=round(c, 4),
                           speedup=round(base["ms"] / rec["ms"], 4), ws_bytes=16 * N * N,
                           ws_over_L2=round(16 * N * N / L2_BYTES, 4), ws_over_MALL=round(16 * N * N / MALL_BYTES, 4))
                _emit(a.out, rec)


def study_controllers(a):
    R = Runner(a.repeats)
    jac = R.jac
    for N in (1024, 2048, 8192):
        for r in (10.0, 100.0):
            steps = 10 if N <= 2048 else 2
            base = dict(kernel=jac.JAC_ASYNC, tile_x=32, tile_y=8, checks=jac.JAC_CHECKS_BLOCKING)
            runs = [(f"static_D{D}", dict(base, D=D)) for D in (1, 2, 4, 8)]
            runs += [("G-asc", dict(base, D=8, controller=jac.JAC_G_ASC)),
                     ("G-desc", dict(base, D=8, controller=jac.JAC_G_DESC)),
                     ("G-fb", dict(base, D=8, controller=jac.JAC_G_FB)),
                     ("sync_overlapped", dict(kernel=jac.JAC_SYNC)),
                     ("temporal_D8_overlapped", dict(kernel=jac.JAC_TBLOCK, D=8))]
            for name, o in runs:
                rec = R.run(N, r, steps, **o)
                rec.update(study="controllers", policy=name)
                _emit(a.out, rec)


def study_overlap(a):
    R = Runner(a.repeats)
    jac = R.jac
    for N in (2048, 8192):
        for D, tx, ty in ((8, 32, 16), (8, 64, 16), (16, 64, 32)):
            for o in (0, 1, 2, 4, D - 1):
                if (tx + 2 * o) * (ty + 2 * o) > 4096:
                    continue
                rec = R.run(N, 10.0, 10 if N <= 2048 else 2, kernel=jac.JAC_ASYNC, D=D, M=8, tile_x=tx, tile_y=ty,
                            overlap=o)
                rec.update(study="overlap", D=D, tile=[tx, ty], overlap=o)
                _emit(a.out, rec)


# MI355X: 8 TB/s of HBM; 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz non-packed float32 lane-operations.
HBM_PEAK = 8.0e12
VALU_PEAK = 256 * 4 * 16 * 2.4e9


def _launch_profile(R, N, r, steps, kclass, every, **o):
    """Mean device time (us) of the launches of one class over a profiled solve."""
    sol = R.solver(N, r)
    opts = R.jac.jac_opts_default(**o)
    sol.reset()
    sol.profile(every)
    sol.solve(steps, opts)
    R.torch.cuda.synchronize()
    avg_ms, n, nt = sol.profile_read(kclass)
    sol.profile(0)
    return 1e3 * avg_ms, n, nt


def study_depths(a):
    R = Runner(a.repeats)
    jac = R.jac
    N, r, steps = 8192, 10.0, 10
    base = R.run(N, r, steps, kernel=jac.JAC_SYNC)
    base.update(study="depths", family="sync", D=1, s=1.0, c=1.0)
    _emit(a.out, base)
    fams = (("temporal", jac.JAC_TBLOCK, "tblock"), ("async_32x16", jac.JAC_ASYNC, "async"))
    for fam, kernel, kc in fams:
        if a.family != "all" and not fam.startswith(a.family):
            continue
        for D in range(1, 17):
            o = dict(kernel=kernel, D=D, tile_x=32, tile_y=16)
            rec = R.run(N, r, steps, **o)
            # per-launch time of launches of D sweeps: below 9, from a solve checking
            # every D sweeps (with M = 8 a depth that does not divide 8 also issues
            # shorter launches to reach each check); from 9 on, temporal blocking's
            # own solve (its launches of D sweeps check inner levels; shorter ones
            # have a class of their own), block-async checking every D
            deep = kernel == jac.JAC_TBLOCK and D >= 9
            us, n, nt = _launch_profile(R, N, r, steps, kc, 8, **(o if deep else dict(o, M=max(D, 1))))
            upd = D * N * N  # point-updates per launch of D sweeps
            rec.update(study="depths", family=fam, D=D,
                       interval=8 if kernel == jac.JAC_TBLOCK else max(8, D),
                       s=round(rec["sweeps"] / base["sweeps"], 4),
                       c=round((rec["ms"] / rec["sweeps"]) / (base["ms"] / base["sweeps"]), 4),
                       launch_us=round(us, 2), launches=n, timed=nt,
                       hbm_frac=round(12.0 * N * N / (us * 1e-6) / HBM_PEAK, 4),
                       valu_frac=round(8.0 * upd / (us * 1e-6) / VALU_PEAK, 4),
                       exact_gpts=round(N * N * base["sweeps"] / (rec["ms"] / 1e3) / 1e9, 1))
            _emit(a.out, rec)


def study_launches(a):
    R = Runner(a.repeats)
    jac = R.jac
    cases = [("sync", "sync_check", dict(kernel=jac.JAC_SYNC)),
             ("async_D1_32x16", "async", dict(kernel=jac.JAC_ASYNC, D=1, tile_x=32, tile_y=16)),
             ("async_D8_32x16", "async", dict(kernel=jac.JAC_ASYNC, D=8, tile_x=32, tile_y=16)),
             ("temporal_D8", "tblock", dict(kernel=jac.JAC_TBLOCK, D=8))]
    for N in (256, 512, 1024):
        for name, kc, o in cases:
            for driver in (jac.JAC_LAUNCH, jac.JAC_GRAPH, jac.JAC_PERSISTENT):
                rec = R.run(N, 10.0, 10, driver=driver, **o)
                D = o.get("D", 1)
                launches = rec["sweeps"] / D
                rec.update(study="launches", case=name, driver=["launch", "graph", "persistent"][driver],
                           wall_us_per_launch=round(rec["ms"] * 1e3 / launches, 2),
                           wall_us_per_sweep=rec["us_per_sweep"])
                if driver == jac.JAC_LAUNCH:
                    us = []
                    for _ in range(max(5, a.repeats)):
                        u, n, nt = _launch_profile(R, N, 10.0, 10, kc, 1, driver=driver, **o)
                        us.append(u)
                    rec.update(device_us_per_launch=round(statistics.median(us), 2), device_repeats=len(us))
                    if kc == "sync_check":  # the other synchronous launches carry no check
                        us = [_launch_profile(R, N, 10.0, 10, "sync", 1, driver=driver, **o)[0]
                              for _ in range(max(5, a.repeats))]
                        rec.update(device_us_per_plain_sweep=round(statistics.median(us), 2))
                _emit(a.out, rec)


def fit(a):
    """Depth-2 tree on (ws / L2, r) -> fastest family, leave-one-size-out."""
    from sklearn.tree import DecisionTreeClassifier, export_text

    rows = [json.loads(l) for l in open(a.regimes) if l.strip()]
    rows = [x for x in rows if x.get("study") == "regimes"]
    fam = {"sync": "sync", "temporal_D4": "temporal", "temporal_D8": "temporal",
           "async_D4_32x8": "staleness", "async_D8_32x16": "staleness"}
    best = {}
    for x in rows:
        if x["family"] not in fam:
            continue
        key = (x["N"], x["r"])
        if key not in best or x["ms"] < best[key]["ms"]:
            best[key] = x
    keys = sorted(best)
    X = [[best[k]["ws_over_L2"], k[1]] for k in keys]
    y = [fam[best[k]["family"]] for k in keys]
    tree = DecisionTreeClassifier(max_depth=2, random_state=0).fit(X, y)
    print(export_text(tree, feature_names=["ws_over_L2", "r"]))
    hits = 0
    for n in sorted({k[0] for k in keys}):
        tr = [i for i, k in enumerate(keys) if k[0] != n]
        te = [i for i, k in enumerate(keys) if k[0] == n]
        t = DecisionTreeClassifier(max_depth=2, random_state=0).fit([X[i] for i in tr], [y[i] for i in tr])
        hits += sum(t.predict([X[i]])[0] == y[i] for i in te)
    print(f"leave-one-size-out: {hits}/{len(keys)} configurations predicted")
    for k, lab in zip(keys, y):
        print(f"N={k[0]:6d} r={k[1]:5.0f}  fastest {best[k]['family']:16s} ({lab})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("study", choices=("checks", "regimes", "controllers", "overlap", "depths", "launches", "fit"))
    ap.add_argument("regimes", nargs="?", help="fit: the regimes study's JSON lines")
    ap.add_argument("--out", default=None)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--family", choices=("all", "temporal", "async"), default="all",
                    help="depths: the strategy families to run")
    a = ap.parse_args()
    {"checks": study_checks, "regimes": study_regimes, "controllers": study_controllers,
     "overlap": study_overlap, "depths": study_depths, "launches": study_launches, "fit": fit}[a.study](a)


if __name__ == "__main__":
    main()
