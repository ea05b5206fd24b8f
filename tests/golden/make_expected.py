"""Write the oracle's expected results for the large workloads.

Calls only the CPU oracle (oracle/) and the input generators (workloads.py);
nothing from the HIP library.  For each workload it runs the ten
backward-Euler steps one at a time and stores, per step, the sweep count, the
bit pattern of rho and the SHA-256 of the N x N float32 field (row-major,
little-endian).  The GPU parity tests compare the library's fields against
these hashes bit for bit.

    python -m tests.golden.make_expected C3          # N=8192, r=10, Gaussian
    python -m tests.golden.make_expected C4 --steps 2
    python -m tests.golden.make_expected C3 --mode async --D 8 --tile 32 16
    python -m tests.golden.make_expected C3 --M 12     # temporal blocking at D = 12 checks every 12
    python -m tests.golden.make_expected C3 --mode async --D 4 --tile 32 8 --versus-sync

--versus-sync (async mode) also runs the synchronous oracle step by step and
stores, per step, max |u_async - u_sync| over ||b_A|| of that step of the
synchronous solve: the block-asynchronous tolerance (final field within
1e-4 ||b_A|| of the exact method's, page "stencil-jacobian.vercel.app",
section 02) measured on the oracle alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def field_hash(u: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(u, dtype="<f4").tobytes()).hexdigest()


def run(name: str, steps: int | None, M: int = 8, mode: str = "sync", D: int = 1, tile=(32, 8),
        versus_sync: bool = False) -> dict:
    cfg = workloads.CONFIGS[name]
    N, r, kind = cfg["N"], cfg["r"], cfg["source"]
    steps = steps or cfg["steps"]
    s = workloads.source(kind, N, r)
    u = np.zeros((N, N), np.float32)
    out = dict(config=name, N=N, r=r, source=kind, M=M, tol=1e-5, steps=steps, mode=mode, D=D, tile=list(tile),
               sweeps=[], rho_bits=[], field_sha256=[], oracle_threads=oracle.get_threads(), seconds=[])
    omode = oracle.ASYNC if mode == "async" else oracle.SYNC
    if versus_sync:
        out.update(sync_sweeps=[], bA_sync=[], max_diff_vs_sync=[], max_diff_over_bA=[])
        us = np.zeros((N, N), np.float32)
    for n in range(steps):
        t0 = time.time()
        res = oracle.solve(N, r, s, u0=u, steps=1, M=M, mode=omode, D=D, tx=tile[0], ty=tile[1])
        if res.status != oracle.OK:
            raise RuntimeError(f"{name} step {n}: oracle status {res.status}")
        u = res.u
        if versus_sync:
            bA = float(oracle.rhs_norm(oracle.rhs(us, s), r))
            ref = oracle.solve(N, r, s, u0=us, steps=1, M=M, mode=oracle.SYNC)
            if ref.status != oracle.OK:
                raise RuntimeError(f"{name} step {n}: synchronous oracle status {ref.status}")
            us = ref.u
            diff = float(np.max(np.abs(u.astype(np.float64) - us.astype(np.float64))))
            out["sync_sweeps"].append(int(ref.sweeps[0]))
            out["bA_sync"].append(bA)
            out["max_diff_vs_sync"].append(diff)
            out["max_diff_over_bA"].append(diff / bA)
            print(f"  versus sync: max diff {diff:.4e} = {diff / bA:.4e} ||b_A||", flush=True)
        out["sweeps"].append(int(res.sweeps[0]))
        out["rho_bits"].append(f"{np.float32(res.rho[0]).view(np.uint32):08x}")
        out["field_sha256"].append(field_hash(u))
        out["seconds"].append(round(time.time() - t0, 2))
        print(f"{name} step {n}: sweeps {res.sweeps[0]} rho {res.rho[0]:.6e} ({out['seconds'][-1]} s)", flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("config")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--mode", choices=("sync", "async"), default="sync")
    ap.add_argument("--D", type=int, default=1)
    ap.add_argument("--tile", type=int, nargs=2, default=(32, 8))
    ap.add_argument("--M", type=int, default=8, help="check interval (async: the interval is max(M, D))")
    ap.add_argument("--versus-sync", action="store_true")
    ap.add_argument("--threads", type=int, default=0, help="oracle threads (0: all)")
    args = ap.parse_args()
    if args.threads > 0:
        oracle.set_threads(args.threads)
    res = run(args.config, args.steps, M=args.M, mode=args.mode, D=args.D, tile=tuple(args.tile),
              versus_sync=args.versus_sync)
    tag = args.config if args.mode == "sync" else f"{args.config}_async_D{args.D}_{args.tile[0]}x{args.tile[1]}"
    if args.M != 8:
        tag += f"_M{args.M}"
    path = os.path.join(HERE, f"expected_{tag}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
