/*
 * jacobi_oracle.c -- plain CPU reference for the backward-Euler five-point
 * Jacobi solve ("the oracle").
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may include, link
 * or call this file: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no header, helper or constant with the
 * HIP sources of jacobi_stencil_amd/.
 *
 * What it computes (page "stencil-jacobian.vercel.app", section 01 "The
 * problem" and section 02 "Method"):
 *   - The transient equation du/dt = alpha*lap(u) + f on an N x N grid of
 *     unknowns, one backward-Euler step at a time.  With r = alpha*dt/h^2 each
 *     step solves  (1+4r) u - r (uE+uW+uN+uS) = b,  b = u^n + dt*f, with u^n
 *     held fixed during the step.  The top boundary is held at 100, the other
 *     three sides at 0.
 *   - Point Jacobi: u' = (b + r (uE+uW+uN+uS)) / (1+4r), every point from the
 *     previous iterate.
 *   - Stop when rho = ||b_A - A u||_inf / ||b_A||_inf < tol, tested every M
 *     sweeps on the newest iterate, with the residual in difference form.
 *   - Block-asynchronous variant (same page, section 02, after Anzt et al.;
 *     also Islam & Wang, "Hierarchical Jacobi Iteration ... using Shared
 *     Memory", section 3): each tile copies itself plus a one-cell halo, the
 *     halo stays frozen, D Jacobi sweeps run on the tile, the tile is written
 *     back.
 *
 * Arithmetic (same page, section 02: round-to-nearest single-precision
 * operations, no fused multiply-add, one fixed order).  Every operation below
 * is one IEEE-754 binary32 operation; the file must be compiled with
 * -ffp-contract=off and without -ffast-math so that nothing is fused,
 * reassociated or flushed to zero.  The readings of the page that fix the
 * order where it is silent:
 *   sweep:    S = ((uE + uW) + uN) + uS;  u' = (b + r*S) / d,  d = 1 + 4r
 *   residual: C = u;  e = (((uE-C) + (uW-C)) + (uN-C)) + (uS-C);
 *             res = (b - C) + r*e;  R = max |res|  (NaN wins)
 *   norm:     bA = max |b + r*g|, g = 100 on the row next to the top boundary
 *             and 0 elsewhere (the boundary data moved to the right-hand side)
 *   decision: rho = R / bA;  converged iff rho < tol.
 *
 * Storage: an (N+2) x (N+2) row-major array per buffer.  Row 0 and row N+1,
 * column 0 and column N+1 are the ghost ring, written once: the top row
 * (next to unknown row 0) holds 100, the rest 0.  Unknown (i, j), i = row from
 * the top, j = column, lives at (i+1, j+1).  Arrays handed in and out are the
 * N x N unknowns only, row-major.
 *
 * The loops over rows carry OpenMP pragmas; every point update is independent
 * and max is exact, so the result does not depend on the thread count.
 */
#include "jacobi_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TOP_VALUE 100.0f

static size_t pitch_of(int N) { return (size_t)N + 2; }
static size_t at(int N, int i, int j) { return (size_t)(i + 1) * pitch_of(N) + (size_t)(j + 1); }

/* Ghost ring of a padded buffer: top row 100, other sides 0, corners 0. */
static void set_ghosts(int N, float* U) {
    size_t P = pitch_of(N);
    for (size_t j = 0; j < P; ++j) { U[j] = 0.0f; U[(size_t)(N + 1) * P + j] = 0.0f; }
    for (int j = 0; j < N; ++j) U[at(N, -1, j)] = TOP_VALUE;
    for (int i = -1; i <= N; ++i) { U[at(N, i, -1)] = 0.0f; U[at(N, i, N)] = 0.0f; }
}

static float* alloc_padded(int N) {
    size_t n = pitch_of(N) * pitch_of(N);
    float* p = (float*)calloc(n, sizeof(float));
    if (p) set_ghosts(N, p);
    return p;
}

static void load_interior(int N, float* U, const float* src) {
    for (int i = 0; i < N; ++i) memcpy(&U[at(N, i, 0)], &src[(size_t)i * N], (size_t)N * sizeof(float));
}

static void store_interior(int N, const float* U, float* dst) {
    for (int i = 0; i < N; ++i) memcpy(&dst[(size_t)i * N], &U[at(N, i, 0)], (size_t)N * sizeof(float));
}

/* d = 1 + 4r, two rounded operations. */
static float diag_of(float r) {
    float four_r = 4.0f * r;
    return 1.0f + four_r;
}

/* One point of the Jacobi update from a padded buffer. */
static float jacobi_point(const float* U, size_t c, size_t P, float b, float r, float d) {
    float uE = U[c + 1], uW = U[c - 1], uN = U[c - P], uS = U[c + P];
    float S = uE + uW;
    S = S + uN;
    S = S + uS;
    float t = r * S;
    float n = b + t;
    return n / d;
}

/* One point of the difference-form residual b_A - A u. */
static float residual_point(const float* U, size_t c, size_t P, float b, float r) {
    float C = U[c];
    float e = (U[c + 1] - C) + (U[c - 1] - C);
    e = e + (U[c - P] - C);
    e = e + (U[c + P] - C);
    float bc = b - C;
    float t = r * e;
    return bc + t;
}

/* ---- single operations on padded buffers ------------------------------- */

static void rhs_padded(int N, const float* U, const float* s, float* B) {
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) B[at(N, i, j)] = U[at(N, i, j)] + s[(size_t)i * N + j];
}

static float rhs_norm_padded(int N, float r, const float* B) {
    float m = 0.0f;
    int nan_seen = 0;
    #pragma omp parallel for schedule(static) reduction(max : m) reduction(| : nan_seen)
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            float g = (i == 0) ? TOP_VALUE : 0.0f;
            float v = B[at(N, i, j)] + r * g;
            float a = fabsf(v);
            if (isnan(a)) nan_seen = 1;
            else if (a > m) m = a;
        }
    return nan_seen ? NAN : m;
}

static void sweep_padded(int N, float r, float d, const float* U, const float* B, float* V) {
    size_t P = pitch_of(N);
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            size_t c = at(N, i, j);
            V[c] = jacobi_point(U, c, P, B[c], r, d);
        }
}

static float residual_padded(int N, float r, const float* U, const float* B) {
    size_t P = pitch_of(N);
    float m = 0.0f;
    int nan_seen = 0;
    #pragma omp parallel for schedule(static) reduction(max : m) reduction(| : nan_seen)
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            size_t c = at(N, i, j);
            float a = fabsf(residual_point(U, c, P, B[c], r));
            if (isnan(a)) nan_seen = 1;
            else if (a > m) m = a;
        }
    return nan_seen ? NAN : m;
}

/*
 * One block-asynchronous launch.  Tiles of tx columns by ty rows start at the
 * top-left unknown; the last tile in each direction may be partial.  Each tile
 * owns its points.  It works on its points widened by o cells on each side
 * (clipped to the grid): the overlapping subdomains of Islam & Wang,
 * "Hierarchical Jacobi Iteration ... using Shared Memory", section 3.5 (1-D)
 * and the 2-D extension in section 4; o = 0 is the plain block-async launch of
 * page "stencil-jacobian.vercel.app", section 02.  It copies that region and
 * the one-cell ring around it from U (the ring holds neighbouring tiles'
 * values or the ghost ring, and stays frozen), performs D Jacobi sweeps on the
 * region, each sweep reading the region's previous sweep, and writes only its
 * own points to V; the values computed in the overlap are dropped.
 */
static void async_launch_padded(int N, float r, float d, const float* U, const float* B, float* V,
                                int tx, int ty, int D, int o) {
    int ntx = (N + tx - 1) / tx, nty = (N + ty - 1) / ty;
    #pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < ntx * nty; ++t) {
        int x0 = (t % ntx) * tx, y0 = (t / ntx) * ty;
        int x1 = (x0 + tx <= N) ? x0 + tx : N;   /* owned columns [x0, x1) */
        int y1 = (y0 + ty <= N) ? y0 + ty : N;   /* owned rows [y0, y1) */
        int ex0 = x0 - o < 0 ? 0 : x0 - o, ex1 = x1 + o > N ? N : x1 + o;
        int ey0 = y0 - o < 0 ? 0 : y0 - o, ey1 = y1 + o > N ? N : y1 + o;
        int w = ex1 - ex0, h = ey1 - ey0;          /* the region worked on */
        size_t lp = (size_t)w + 2;
        size_t ln = lp * ((size_t)h + 2);
        float* cur = (float*)malloc(ln * sizeof(float));
        float* nxt = (float*)malloc(ln * sizeof(float));
        float* bl = (float*)malloc(ln * sizeof(float));
        /* local (a, c) with a = 0..h+1, c = 0..w+1 is unknown (ey0+a-1, ex0+c-1) */
        for (int a = 0; a < h + 2; ++a)
            for (int c = 0; c < w + 2; ++c) {
                size_t g = at(N, ey0 + a - 1, ex0 + c - 1);
                cur[(size_t)a * lp + c] = U[g];
                bl[(size_t)a * lp + c] = B[g];
            }
        memcpy(nxt, cur, ln * sizeof(float));
        for (int sweep = 0; sweep < D; ++sweep) {
            for (int a = 1; a <= h; ++a)
                for (int c = 1; c <= w; ++c) {
                    size_t l = (size_t)a * lp + c;
                    nxt[l] = jacobi_point(cur, l, lp, bl[l], r, d);
                }
            float* tmp = cur; cur = nxt; nxt = tmp;
        }
        for (int i = y0; i < y1; ++i)
            for (int j = x0; j < x1; ++j)
                V[at(N, i, j)] = cur[(size_t)(i - ey0 + 1) * lp + (size_t)(j - ex0 + 1)];
        free(cur); free(nxt); free(bl);
    }
}

/* ---- exported single operations (N x N unknowns in and out) ------------ */

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

float orc_diag(float r) { return diag_of(r); }

void orc_rhs(int N, const float* u, const float* s, float* b) {
    float* U = alloc_padded(N);
    float* B = alloc_padded(N);
    load_interior(N, U, u);
    rhs_padded(N, U, s, B);
    store_interior(N, B, b);
    free(U); free(B);
}

float orc_rhs_norm(int N, float r, const float* b) {
    float* B = alloc_padded(N);
    load_interior(N, B, b);
    float m = rhs_norm_padded(N, r, B);
    free(B);
    return m;
}

void orc_sweep(int N, float r, const float* u, const float* b, float* out) {
    float* U = alloc_padded(N);
    float* B = alloc_padded(N);
    float* V = alloc_padded(N);
    load_interior(N, U, u);
    load_interior(N, B, b);
    sweep_padded(N, r, diag_of(r), U, B, V);
    store_interior(N, V, out);
    free(U); free(B); free(V);
}

float orc_residual(int N, float r, const float* u, const float* b) {
    float* U = alloc_padded(N);
    float* B = alloc_padded(N);
    load_interior(N, U, u);
    load_interior(N, B, b);
    float m = residual_padded(N, r, U, B);
    free(U); free(B);
    return m;
}

void orc_async_launch(int N, float r, const float* u, const float* b, float* out, int tx, int ty, int D, int o) {
    float* U = alloc_padded(N);
    float* B = alloc_padded(N);
    float* V = alloc_padded(N);
    load_interior(N, U, u);
    load_interior(N, B, b);
    async_launch_padded(N, r, diag_of(r), U, B, V, tx, ty, D, o);
    store_interior(N, V, out);
    free(U); free(B); free(V);
}

/* ---- the time-step loop -------------------------------------------------- */

/*
 * Depth chosen by the threshold controllers of page "stencil-jacobian.vercel.
 * app", section 02 (block-async, "G-asc and G-desc"): the depth steps as rho
 * crosses 1e-2, 1e-3 and 1e-4.  Reading of the page: three thresholds give
 * four depths, 1, 2, 4 and 8.  G-asc starts each time step at D = 1 and moves
 * through 1, 2, 4, 8 as rho falls below each threshold; G-desc starts at 8 and
 * moves through 8, 4, 2, 1.  Each depth is capped at Dmax (min(level, Dmax):
 * with Dmax = 6 G-desc runs 6, 4, 2, 1 and G-asc 1, 2, 4, 6; with Dmax = 16
 * neither goes past 8).  Both are latched: within a time step the depth never
 * moves back.  rho is compared with the thresholds as binary32 values.
 */
static int asc_level(float q) {
    if (q >= 1e-2f) return 1;
    if (q >= 1e-3f) return 2;
    if (q >= 1e-4f) return 4;
    return 8;
}
static int desc_level(float q) {
    if (q >= 1e-2f) return 8;
    if (q >= 1e-3f) return 4;
    if (q >= 1e-4f) return 2;
    return 1;
}
static int cap_depth(int level, int Dmax) { return level > Dmax ? Dmax : level; }

/*
 * Ten (or `steps`) backward-Euler steps, each iterated to rho < tol.
 *   u_io:    in: u^0 (N x N); out: the last field.
 *   mode:    ORC_SYNC  - point Jacobi, a check after every M sweeps;
 *            ORC_ASYNC - block-async launches of min(D, left) sweeps, tiles
 *                        tx x ty widened by o overlap cells; the check
 *                        interval is M, or Dmax when Dmax > M;
 *            ORC_WRONG_B - the mistake page "stencil-jacobian.vercel.app"
 *                        section 01 recounts: point Jacobi with b formed
 *                        from the current iterate before every sweep (and
 *                        the check on that b) instead of from u^n, which
 *                        solves the steady-state problem instead (a negative
 *                        control: its sweep count grows as N^2).
 *   ctrl:    (ORC_ASYNC) how the depth D of each check interval is chosen:
 *            ORC_STATIC D = Dmax throughout; ORC_G_ASC / ORC_G_DESC from the
 *            rho of the previous check (see asc_level / desc_level); ORC_SCHED
 *            the i-th interval of the whole solve uses sched[i] (an interval
 *            beyond sched_n is an error).
 *   sweeps, rho: per-step sweep count and the rho of the accepted iterate.
 *   R_log:   optional; R of every check in order (at most log_cap entries);
 *            *log_n receives the number of checks made.
 *   d_log:   optional; the depth of every interval (at most log_cap entries).
 * Returns ORC_OK, ORC_ENOCONV (a failed check at or beyond max_sweeps: the
 * field is that checked iterate) or ORC_ENAN (rho is NaN: the field is that
 * iterate).  Steps after a failure are not run; their entries are 0 / NaN.
 */
int orc_solve_ex(int N, float r, const float* s, float* u_io, int steps, float tol, int M, int mode,
                 int Dmax, int tx, int ty, int o, int ctrl, const int* sched, int64_t sched_n,
                 int64_t max_sweeps, int64_t* sweeps, float* rho,
                 float* R_log, int* d_log, int64_t log_cap, int64_t* log_n) {
    if (N < 1 || steps < 0 || M < 1 || Dmax < 1 || tx < 1 || ty < 1 || o < 0 || max_sweeps < 1)
        return ORC_EINVAL;
    if (mode != ORC_SYNC && mode != ORC_ASYNC && mode != ORC_WRONG_B) return ORC_EINVAL;
    if (ctrl < ORC_STATIC || ctrl > ORC_SCHED || (ctrl == ORC_SCHED && !sched)) return ORC_EINVAL;
    if (mode != ORC_ASYNC && ctrl != ORC_STATIC) return ORC_EINVAL;
    float d = diag_of(r);
    float* U0 = alloc_padded(N);
    float* U1 = alloc_padded(N);
    float* B = alloc_padded(N);
    if (!U0 || !U1 || !B) { free(U0); free(U1); free(B); return ORC_ENOMEM; }
    load_interior(N, U0, u_io);
    for (int n = 0; n < steps; ++n) { sweeps[n] = 0; rho[n] = NAN; }
    int64_t nlog = 0;
    int status = ORC_OK;
    int interval = (mode == ORC_ASYNC && Dmax > M) ? Dmax : M;
    float* cur = U0;
    float* nxt = U1;
    for (int n = 0; n < steps && status == ORC_OK; ++n) {
        /* right-hand side from u^n, which is also the first iterate */
        rhs_padded(N, cur, s, B);
        float bA = rhs_norm_padded(N, r, B);
        int64_t k = 0;
        int D = Dmax;
        if (ctrl == ORC_G_ASC) D = 1;
        if (ctrl == ORC_G_DESC) D = cap_depth(8, Dmax);
        for (;;) {
            if (ctrl == ORC_SCHED) {
                if (nlog >= sched_n) { status = ORC_EINVAL; break; }
                D = sched[nlog];
                if (D < 1) { status = ORC_EINVAL; break; }
            }
            if (d_log && nlog < log_cap) d_log[nlog] = D;
            int left = interval;
            while (left > 0) {
                if (mode == ORC_SYNC) {
                    sweep_padded(N, r, d, cur, B, nxt);
                    left -= 1;
                } else if (mode == ORC_WRONG_B) {
                    rhs_padded(N, cur, s, B);
                    sweep_padded(N, r, d, cur, B, nxt);
                    left -= 1;
                } else {
                    int m = D < left ? D : left;
                    async_launch_padded(N, r, d, cur, B, nxt, tx, ty, m, o);
                    left -= m;
                }
                float* tmp = cur; cur = nxt; nxt = tmp;
            }
            k += interval;
            if (mode == ORC_WRONG_B) {
                rhs_padded(N, cur, s, B);
                bA = rhs_norm_padded(N, r, B);
            }
            float R = residual_padded(N, r, cur, B);
            float q = R / bA;
            if (R_log && nlog < log_cap) R_log[nlog] = R;
            ++nlog;
            sweeps[n] = k;
            rho[n] = q;
            if (q < tol) break;
            if (isnan(q)) { status = ORC_ENAN; break; }
            if (k >= max_sweeps) { status = ORC_ENOCONV; break; }
            if (ctrl == ORC_G_ASC) {
                int t = cap_depth(asc_level(q), Dmax);
                if (t > D) D = t;
            } else if (ctrl == ORC_G_DESC) {
                int t = cap_depth(desc_level(q), Dmax);
                if (t < D) D = t;
            }
        }
    }
    store_interior(N, cur, u_io);
    if (log_n) *log_n = nlog;
    free(U0); free(U1); free(B);
    return status;
}

int orc_solve(int N, float r, const float* s, float* u_io, int steps, float tol, int M, int mode,
              int D, int tx, int ty, int64_t max_sweeps, int64_t* sweeps, float* rho,
              float* R_log, int64_t log_cap, int64_t* log_n) {
    return orc_solve_ex(N, r, s, u_io, steps, tol, M, mode, D, tx, ty, 0, ORC_STATIC, NULL, 0, max_sweeps,
                        sweeps, rho, R_log, NULL, log_cap, log_n);
}
