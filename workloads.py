"""Synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no arithmetic of the method: it only writes the source term
s = dt*f (an input array) and seeded random fields, as float32 numpy arrays.
Both the HIP library and the CPU oracle receive the same arrays from here.

Problem set-up (page "stencil-jacobian.vercel.app", section 01 "The
problem"): an N x N unit square, ten backward-Euler steps, the source a point
at the centre or a Gaussian of width sigma = N/16.  The page leaves alpha, h
and dt open; the reading used here is alpha = 1, h = 1/(N+1), dt = r*h^2, so
dt*f = r*h^2*f.  For the point source f = 1/h^2 at the centre cell, hence
s = r there; the Gaussian has amplitude 1 and is centred at (N-1)/2.
"""
from __future__ import annotations

import numpy as np


def point_source(N: int, r: float) -> np.ndarray:
    """s = dt*f with f = 1/h^2 on unknown (N//2, N//2), 0 elsewhere: s = r there."""
    s = np.zeros((N, N), np.float32)
    s[N // 2, N // 2] = np.float32(r)
    return s


def gaussian_source(N: int, r: float, sigma: float | None = None) -> np.ndarray:
    """s = dt*f with f = exp(-((i-c)^2 + (j-c)^2) / (2 sigma^2)), c = (N-1)/2.

    Evaluated in float64 and rounded once to float32, so the array is exactly
    left-right (and top-bottom) symmetric.
    """
    if sigma is None:
        sigma = N / 16.0
    h = 1.0 / (N + 1)
    c = (N - 1) / 2.0
    x = (np.arange(N, dtype=np.float64) - c) ** 2
    # One exponent per point, of (x_i + x_j): symmetric under i <-> j and
    # j <-> N-1-j bit for bit.
    f = np.exp(-(x[:, None] + x[None, :]) / (2.0 * sigma * sigma))
    return (float(r) * h * h * f).astype(np.float32)


def source(kind: str, N: int, r: float) -> np.ndarray:
    if kind == "point":
        return point_source(N, r)
    if kind == "gaussian":
        return gaussian_source(N, r)
    if kind == "zero":
        return np.zeros((N, N), np.float32)
    raise ValueError(f"unknown source kind {kind!r}")


def random_source(N: int, r: float, seed: int) -> np.ndarray:
    """Uniform s in [0, r) from numpy's PCG64 with the given seed."""
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.random((N, N)) * float(r)).astype(np.float32)


def random_field(N: int, seed: int, hi: float = 100.0) -> np.ndarray:
    """Uniform u in [0, hi) from numpy's PCG64 with the given seed."""
    g = np.random.Generator(np.random.PCG64(seed + 1_000_003))
    return (g.random((N, N)) * float(hi)).astype(np.float32)


# The five measured workloads: grid size, coupling r, source, what each probes.
CONFIGS = {
    "C1": dict(N=512, r=1.0, source="point", steps=10,
               note="L2-resident, launch-bound"),
    "C2": dict(N=2048, r=10.0, source="gaussian", steps=10,
               note="inside the 256 MB last-level cache; sync vs temporal blocking"),
    "C3": dict(N=8192, r=10.0, source="gaussian", steps=10,
               note="HBM-bound: three arrays of 268 MB"),
    "C4": dict(N=18432, r=100.0, source="point", steps=10,
               note="largest grid; ~1417 sweeps per step"),
    "C5": dict(N=256, r=(1.0, 10.0), source="gaussian", steps=10,
               note="launch-bound; per-sweep launches vs graph vs persistent"),
}
