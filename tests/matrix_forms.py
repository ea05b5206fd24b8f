"""Independent float64 formulations of the linear system, for pinning the oracle.

These do not follow the oracle's loops: they assemble the backward-Euler
matrix A and the boundary-augmented right-hand side b_A of page
"stencil-jacobian.vercel.app", section 01, explicitly (dense or through the
sine transform that diagonalises A) and work in float64.
"""
from __future__ import annotations

import numpy as np
from scipy import fft

TOP = 100.0


def boundary_rhs(b, r):
    """b_A = b + r*g: the Dirichlet data (top 100, others 0) moved to the right-hand side."""
    bA = np.asarray(b, np.float64).copy()
    bA[0, :] += float(r) * TOP
    return bA


def dense_matrix(N, r):
    """A = (1+4r) I - r * (adjacency of the N x N five-point grid), unknown p = i*N + j."""
    n = N * N
    A = np.zeros((n, n))
    r = float(r)
    for i in range(N):
        for j in range(N):
            p = i * N + j
            A[p, p] = 1.0 + 4.0 * r
            for di, dj in ((0, 1), (0, -1), (1, 0), (-1, 0)):
                ii, jj = i + di, j + dj
                if 0 <= ii < N and 0 <= jj < N:
                    A[p, ii * N + jj] = -r
    return A


def apply_A(u, r):
    """A u for the N x N grid with zero outside (shift-based, float64)."""
    u = np.asarray(u, np.float64)
    r = float(r)
    nb = np.zeros_like(u)
    nb[:, :-1] += u[:, 1:]
    nb[:, 1:] += u[:, :-1]
    nb[:-1, :] += u[1:, :]
    nb[1:, :] += u[:-1, :]
    return (1.0 + 4.0 * r) * u - r * nb


def true_residual(u, b, r):
    """max |b_A - A u| in float64."""
    return float(np.max(np.abs(boundary_rhs(b, r) - apply_A(u, r))))


def dense_solve(b, r):
    N = np.asarray(b).shape[0]
    x = np.linalg.solve(dense_matrix(N, r), boundary_rhs(b, r).ravel())
    return x.reshape(N, N)


def dst_solve(b, r):
    """Exact solve of A u = b_A with the 2-D type-I sine transform.

    A's eigenvectors are sin(p pi (i+1)/(N+1)) sin(q pi (j+1)/(N+1)) with
    eigenvalues 1 + 2r (2 - cos(p pi/(N+1)) - cos(q pi/(N+1))).
    """
    N = np.asarray(b).shape[0]
    k = np.arange(1, N + 1)
    c = np.cos(k * np.pi / (N + 1))
    lam = 1.0 + 2.0 * float(r) * (2.0 - c[:, None] - c[None, :])
    bh = fft.dstn(boundary_rhs(b, r), type=1, norm="ortho")
    return fft.idstn(bh / lam, type=1, norm="ortho")


def block_async_launch(u, b, r, tx, ty, D, o=0):
    """One block-asynchronous launch in float64, written as per-tile Jacobi on a local system.

    For each tile T, let E be T widened by o cells per side (clipped to the
    grid): x <- (b_E + r*(Adj_EE x + c_E)) / (1+4r), D times, x0 = u_E, where
    c_E collects the frozen neighbours outside E (other tiles' values of u, or
    the boundary data); only T's points are written back.
    """
    u = np.asarray(u, np.float64)
    bA = boundary_rhs(b, r)
    N = u.shape[0]
    r = float(r)
    out = np.empty_like(u)
    for y0 in range(0, N, ty):
        for x0 in range(0, N, tx):
            own = [(i, j) for i in range(y0, min(y0 + ty, N)) for j in range(x0, min(x0 + tx, N))]
            ys = range(max(y0 - o, 0), min(y0 + ty + o, N))
            xs = range(max(x0 - o, 0), min(x0 + tx + o, N))
            pts = [(i, j) for i in ys for j in xs]
            index = {p: k for k, p in enumerate(pts)}
            n = len(pts)
            adj = np.zeros((n, n))
            frozen = np.zeros(n)
            for k, (i, j) in enumerate(pts):
                for di, dj in ((0, 1), (0, -1), (1, 0), (-1, 0)):
                    q = (i + di, j + dj)
                    if q in index:
                        adj[k, index[q]] = 1.0
                    elif 0 <= q[0] < N and 0 <= q[1] < N:
                        frozen[k] += u[q]
            rhs = np.array([bA[p] for p in pts]) + r * frozen
            x = np.array([u[p] for p in pts])
            for _ in range(D):
                x = (rhs + r * (adj @ x)) / (1.0 + 4.0 * r)
            for p in own:
                out[p] = x[index[p]]
    return out
