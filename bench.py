"""Benchmark: time-to-solution of ten backward-Euler steps at N = 8192, r = 10.

One bench "step" is one whole solve: reset the field to u^0 = 0, then ten
time steps, each Jacobi-iterated until rho < 1e-5 (checked every 8 sweeps),
everything resident in HBM.  The reported value is Gpoint-updates/s =
N^2 * (sweeps of the exact method) / time-to-solution.  Default kernel: exact
temporal blocking, launches of D = 11 sweeps that measure the residual at the
levels where the checks every 8 sweeps fall.

Beside it, on the same JSON line:
  roofline      the dominant kernel's algorithmic bytes per launch (12 bytes per
                point per HBM pass: read u_k, read b, write u_{k+D}) divided by its
                average launch time, measured with HIP events on the library's
                stream during the timed solves, against MI355X's 8 TB/s;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.
With --pcie the line also carries pcie_inclusive: the same solve with its host
buffers, from jac_create copying the source in to jac_get_field copying the
field out (the workspace already allocated), never the value.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--kernel sync|tblock|async] [--D D]
                       [--config C1..C5] [--driver launch|graph|persistent]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BYTES_PER_POINT_PASS = 12.0    # read u_k, read b, write the next iterate
# non-packed float32 VALU: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# fewest VALU instructions per point-update: 3 adds, 1 mul, 1 add, and the
# verified constant-divisor quotient (1 mul, 2 fma)
VALU_OPS_PER_UPDATE = 8
METRIC = "Gpoint-updates/s + time-to-solution (10 steps), N=8192 r=10; % HBM roofline"
KERNELS = {"sync": 0, "tblock": 1, "async": 2}
DOMINANT_CLASS = {"sync": "sync", "tblock": "tblock", "async": "async"}
DRIVERS = {"launch": 0, "graph": 1, "persistent": 2}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="C3")
    ap.add_argument("--kernel", default="tblock", choices=sorted(KERNELS))
    ap.add_argument("--D", type=int, default=11)
    ap.add_argument("--tile-x", type=int, default=32)
    ap.add_argument("--tile-y", type=int, default=8)
    ap.add_argument("--band-rows", type=int, default=0, help="TBLOCK rows per band (0: automatic)")
    ap.add_argument("--driver", default="launch", choices=sorted(DRIVERS),
                    help="how the launches are issued (the launch-bound sizes compare them)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--profile-every", type=int, default=16,
                    help="bracket every k-th launch of a class with HIP events (0: none)")
    ap.add_argument("--cpu-steps", type=int, default=10, help="time steps in the CPU sample")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: all host cores)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle on the workload and print its cpu_baseline object")
    ap.add_argument("--pcie", action="store_true",
                    help="also time create (source in) + solve + field out through host buffers")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="array size of the bandwidth probe, MiB (0: skip)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files into HBM bytes per launch, then exit")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="summarise rocprofv3 --pmc counter files for the --kernel class "
                         "(median per real launch of its most-called kernel), then exit")
    return ap.parse_args()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, nsteps, threads=0):
    """The oracle on the host cores (all of them, or `threads`), timed on the
    first `nsteps` time steps of the workload."""
    import oracle
    import workloads

    if threads > 0:
        oracle.set_threads(threads)
    N, r = cfg["N"], cfg["r"]
    s = workloads.source(cfg["source"], N, r)
    t0 = time.perf_counter()
    res = oracle.solve(N, r, s, steps=nsteps)
    dt = time.perf_counter() - t0
    sw = int(res.sweeps.sum())
    return {"value": N * N * sw / dt / 1e9, "unit": "Gpoint-updates/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"{cfg['name']} time steps 1-{nsteps} of 10 ({sw} sweeps, {dt:.1f} s), "
                      f"OpenMP over rows, float32",
            "host": {"nproc": os.cpu_count(), "cpu": cpu_model()}}


def copy_probe(torch, jac, mib):
    """Achievable HBM bandwidth from the library's streaming probe (16-byte
    accesses, nontemporal stores): best of copy and add over a few grid sizes,
    each timed with events.  The first launch, a copy of exactly `mib` MiB, is
    also the known-size kernel the memory counters are calibrated against."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.ones_like(a)
    c = torch.empty_like(a)
    st = torch.cuda.current_stream().cuda_stream
    best = {}
    for kind, per_elem in ((0, 8), (1, 12)):
        for blocks in (1024, 65536):
            for _ in range(2):
                jac.jac_stream_probe(c.data_ptr(), a.data_ptr(), b.data_ptr(), n, kind, True, blocks, st)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                jac.jac_stream_probe(c.data_ptr(), a.data_ptr(), b.data_ptr(), n, kind, True, blocks, st)
            e1.record()
            torch.cuda.synchronize()
            gbs = per_elem * n / (e0.elapsed_time(e1) / reps / 1e3) / 1e9
            name = "copy" if kind == 0 else "add"
            best[name] = max(best.get(name, 0.0), gbs)
    del a, b, c
    return {k: round(v, 1) for k, v in best.items()}


def traffic_from(fetch_csv, write_csv, probe_mib, out_path, key):
    """HBM bytes per launch of the dominant kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the probe's copy of a known size."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]) * 1024.0)
        return vals

    fetch = _grouped(per_kernel(fetch_csv, "FETCH_SIZE"))
    write = _grouped(per_kernel(write_csv, "WRITE_SIZE"))
    known = probe_mib * (1 << 20)
    probe = next(k for k in fetch if "k_probe<0" in k)
    f_scale = known / fetch[probe][0]    # the first probe launch is the copy of `probe_mib`
    w_scale = known / write[probe][0]
    pattern = {"tblock": "k_tblock", "async": "k_async", "sync": "k_sync<"}[key.split(":")[1]]
    cands = [k for k in fetch if pattern in k]
    rows = []
    for k in cands:
        fs = [v for v in fetch[k] if v > 1e6]   # launches that returned at once fetch ~nothing
        ws = [v for v in write.get(k, []) if v > 1e6]
        if fs and ws:
            rows.append((len(fs), statistics.median(fs) * f_scale, statistics.median(ws) * w_scale, k))
    rows.sort(reverse=True)
    n, fb, wb, kname = rows[0]
    res = {"kernel": kname, "dispatches": n, "fetch_bytes": fb, "write_bytes": wb,
           "bytes_per_launch": fb + wb, "fetch_scale": f_scale, "write_scale": w_scale,
           "source_sha256": _kernel_source_hash(key.split(":")[1])}
    table = json.load(open(out_path)) if os.path.exists(out_path) else {}
    table[key] = res
    with open(out_path, "w") as f:
        json.dump(table, f, indent=1)
    print(json.dumps({key: res}, indent=1))


def _kernel_group(name):
    """A kernel's name without the compile-time check levels: the deep
    temporal-blocking launches of one depth run as several kernels that differ
    only in the levels they check, with the same data movement."""
    import re

    return re.sub(r"(k_tblock<\d+, \w+, \w+, \w+), -?\d+>", r"\1>", name)


def _grouped(vals):
    out = {}
    for k, v in vals.items():
        out.setdefault(_kernel_group(k), []).extend(v)
    return out


def counters_from(paths, kclass):
    """Median per launch of every counter or derived metric in rocprofv3 --pmc
    files, for the most-called kernel of a class.  Launches queued after a
    stopping check return at once; only launches that ran at least half as
    long as the longest one are counted."""
    import csv
    import statistics

    pattern = {"tblock": "k_tblock", "async": "k_async", "sync": "k_sync<"}[kclass]
    per = {}  # kernel -> dispatch -> (duration ns, {counter: value})
    for path in paths:
        for row in csv.DictReader(open(path)):
            k = _kernel_group(row["Kernel_Name"])
            if pattern not in k:
                continue
            key = (path, row["Dispatch_Id"])
            dur = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            d = per.setdefault(k, {}).setdefault(key, [dur, {}])
            d[1][row["Counter_Name"]] = d[1].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    kname = max(per, key=lambda k: len(per[k]))
    ds = list(per[kname].values())
    longest = max(dur for dur, _ in ds)
    real = [c for dur, c in ds if dur >= longest / 2]
    names = sorted({n for c in real for n in c})
    res = {"kernel": kname, "launches": len(real),
           "median": {n: statistics.median(c[n] for c in real if n in c) for n in names}}
    print(json.dumps(res, indent=1))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the solver runs on a single MI355X "
              "(multi-GPU sharding is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.cpu_only:
        import workloads

        cfg = dict(workloads.CONFIGS[args.config], name=args.config)
        if isinstance(cfg["r"], tuple):
            cfg["r"] = cfg["r"][-1]
        print(json.dumps({"config": args.config, "cpu_baseline": cpu_baseline(cfg, args.cpu_steps, args.cpu_threads)}),
              flush=True)
        return
    # counter-file summaries need no device
    if args.counters_from:
        counters_from(args.counters_from, args.kernel)
        return
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_mib, args.traffic,
                     f"{args.config}:{args.kernel}:D{1 if args.kernel == 'sync' else args.D}")
        return

    import torch

    import jacobi_stencil_amd as jac
    import workloads
    cfg = dict(workloads.CONFIGS[args.config], name=args.config)
    N, r = cfg["N"], cfg["r"]
    if isinstance(r, tuple):
        r = r[-1]
        cfg["r"] = r
    nsteps = cfg["steps"]
    s = workloads.source(cfg["source"], N, r)
    torch.cuda.set_device(0)
    probe = copy_probe(torch, jac, args.copy_mib) if args.copy_mib > 0 else None
    stream = torch.cuda.current_stream()
    sol = jac.Solver(N, r, s, stream=stream)
    opts = jac.jac_opts_default(kernel=KERNELS[args.kernel], D=args.D, tile_x=args.tile_x,
                                tile_y=args.tile_y, band_rows=args.band_rows, driver=DRIVERS[args.driver])

    def one_solve():
        sol.reset()
        return sol.solve(nsteps, opts)

    for _ in range(args.warmup):
        one_solve()
    torch.cuda.synchronize()

    sol.profile(args.profile_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sweeps = None
    for _ in range(args.steps):
        _, sweeps, rho = one_solve()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the persistent driver runs each whole solve as one launch
    cls = "persistent" if args.driver == "persistent" else DOMINANT_CLASS[args.kernel]
    launch_ms, k_n, k_timed = sol.profile_read(cls)
    _, noop_n, _ = sol.profile_read("noop")
    sol.profile(0)

    ms_per_step = elapsed / args.steps * 1e3
    total_sweeps = int(sweeps.sum())
    exact_sweeps = total_sweeps
    if args.kernel == "async":
        # the value counts the exact method's sweeps: take them from an untimed
        # temporally blocked solve of the same workload (bitwise the synchronous one)
        sol.reset()
        _, ex, _ = sol.solve(nsteps, jac.jac_opts_default(kernel=KERNELS["tblock"], D=8))
        exact_sweeps = int(ex.sum())
    value = N * N * exact_sweeps / (ms_per_step / 1e3) / 1e9
    D = 1 if args.kernel == "sync" else args.D
    # one pass over memory per D sweeps; a persistent launch makes all of a solve's passes
    passes_per_launch = total_sweeps / D if args.driver == "persistent" else 1
    bytes_per_launch = BYTES_PER_POINT_PASS * N * N * passes_per_launch
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    traffic = None
    if os.path.exists(args.traffic):
        t = json.load(open(args.traffic))
        key = f"{args.config}:{args.kernel}:D{D}"
        if key in t and t[key].get("source_sha256") == _kernel_source_hash(args.kernel):
            traffic = t[key]["bytes_per_launch"]

    common = {"traffic": traffic, "kernel_class": cls, "launches": k_n, "timed_launches": k_timed,
              "avg_launch_us": round(launch_ms * 1e3, 3), "algorithmic_bytes_per_launch": bytes_per_launch,
              "noop_launches": noop_n}
    hbm = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4)}
    if args.kernel == "sync":
        roofline = dict(hbm, **common)
    else:
        # D sweeps per launch: bound by VALU instruction issue (SQ counters), not by HBM
        tops = N * N * D * passes_per_launch * VALU_OPS_PER_UPDATE / (launch_ms / 1e3) / 1e12
        roofline = dict({"bound": "alu", "achieved": round(tops, 2), "peak": round(VALU_PEAK_TOPS, 2),
                         "unit": "TVALUop/s", "frac": round(tops / VALU_PEAK_TOPS, 4),
                         "valu_ops_per_update": VALU_OPS_PER_UPDATE, "hbm_view": hbm}, **common)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "Gpoint-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: N={N} r={r:g} {cfg['source']} source, {nsteps} backward-Euler "
                               f"steps, Jacobi to rho<1e-5 checked every 8 sweeps",
                   "N": N, "r": r, "source": cfg["source"], "time_steps": nsteps, "kernel": args.kernel,
                   "D": D, "tile": [args.tile_x, args.tile_y] if args.kernel == "async" else None,
                   "driver": args.driver},
        "time_to_solution_ms": round(ms_per_step, 3),
        "sweeps_per_solve": total_sweeps,
        "sweeps_per_step": sweeps.tolist(),
        "exact_sweeps_per_solve": exact_sweeps,
        "extra_sweep_ratio": round(total_sweeps / exact_sweeps, 4),
        "pct_hbm_roofline_model": round(100.0 * value * BYTES_PER_POINT_PASS / D / HBM_PEAK_GBS, 2),
        "stream_probe_gbs": probe,
        "roofline": roofline,
    }
    if args.pcie:
        sol.close()
        line["pcie_inclusive"] = pcie_inclusive(jac, torch, sol, s, nsteps, opts, exact_sweeps)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_steps, args.cpu_threads)
    sol.close()
    print(json.dumps(line), flush=True)


def pcie_inclusive(jac, torch, sol, s, nsteps, opts, exact_sweeps, repeats=3):
    """Whole solves through host buffers on the bench's own workspace: jac_create
    (copies the N x N source in, fills the planes, checks the division), the
    solve, jac_get_field (copies the field out).  Host arrays are touched
    beforehand; median of the repeats."""
    import ctypes
    import statistics

    lib = jac.load_library()
    N = sol.N
    src = np.ascontiguousarray(s, dtype=np.float32)
    out = np.ones((N, N), np.float32)
    rec = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st, h = jac.jac_create(N, sol.r, src, sol.workspace.data_ptr(), sol.ws_bytes, sol.stream.cuda_stream)
        if st != jac.JAC_OK:
            raise RuntimeError(jac.jac_last_error())
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st, _, _ = jac.jac_solve(h, nsteps, opts)
        t2 = time.perf_counter()
        st2 = lib.jac_get_field(h, out.ctypes.data_as(ctypes.c_void_p))
        t3 = time.perf_counter()
        jac.jac_destroy(h)
        if st != jac.JAC_OK or st2 != jac.JAC_OK:
            raise RuntimeError(jac.jac_last_error())
        rec.append((t1 - t0, t2 - t1, t3 - t2, t3 - t0))
    med = [statistics.median(x[i] for x in rec) * 1e3 for i in range(4)]
    return {"value": round(N * N * exact_sweeps / (med[3] / 1e3) / 1e9, 2), "unit": "Gpoint-updates/s",
            "ms": round(med[3], 3), "create_ms": round(med[0], 3), "solve_ms": round(med[1], 3),
            "get_field_ms": round(med[2], 3), "repeats": repeats}


def _kernel_source_hash(kclass):
    """Hash of the sources a kernel class is built from: its own file and the
    shared device header.  Counter figures taken under another hash are stale."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jacobi_stencil_amd", "csrc")
    for f in (f"kernels_{kclass.split('_')[0]}.hip", "jacobi_internal.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


if __name__ == "__main__":
    main()
