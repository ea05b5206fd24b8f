/*
 * jacobi.h -- C interface of libjacobi: backward-Euler implicit diffusion on
 * one MI355X (gfx950), solved step by step with point Jacobi.
 *
 * The method is the one of page "stencil-jacobian.vercel.app":
 *   section 01 "The problem": du/dt = alpha*lap(u) + f on an N x N grid of
 *     unknowns (unit square), ten backward-Euler steps in float32; each step
 *     solves  (1+4r) u - r (uE+uW+uN+uS) = b,  b = u^n + dt*f with u^n held
 *     fixed; the top boundary is held at 100 and the other sides at 0; a step
 *     has converged when rho = ||b_A - A u||_inf / ||b_A||_inf < tol (1e-5),
 *     tested every M (8) sweeps with the residual in difference form.
 *   section 02 "Method": the synchronous sweep (one launch per sweep, fused
 *     right-hand side), the block-asynchronous sweep (tile plus a frozen
 *     one-cell halo, D in-tile sweeps) and exact temporal blocking (a D-cell
 *     ghost zone, D sweeps per pass, identical to D synchronous sweeps); all
 *     arithmetic is round-to-nearest float32 with no fused multiply-add.
 *
 * Readings where the page is silent (the same readings as the test oracle):
 *   - N counts unknowns; u^0 = 0; each step starts from u^n.
 *   - ||b||_inf in rho is the norm of b_A = b + r*g, g = 100 on the top row of
 *     unknowns (the boundary data carried to the right-hand side).
 *   - operation order: S = ((uE+uW)+uN)+uS, u' = (b + r*S)/(1+4r);
 *     e = (((uE-C)+(uW-C))+(uN-C))+(uS-C), res = (b-C) + r*e;
 *     rho = fl(max|res| / ||b_A||).  Subnormals are kept.
 *   - the check after sweeps M, 2M, ... looks at the newest iterate; a step's
 *     sweep count is therefore a multiple of the check interval.
 *
 * Conventions: every array handed across this interface is N x N float32,
 * row-major, row 0 next to the top (100) boundary.  All device work is
 * enqueued on the HIP stream given to jac_create; calls on one context are not
 * thread-safe.  Every function returns a jac_status; the message of the last
 * failure on the calling thread is jac_last_error().
 */
#ifndef LIBJACOBI_H
#define LIBJACOBI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jac_ctx* jac_t;

enum jac_status {
    JAC_OK = 0,
    JAC_EINVAL = -1,   /* bad argument: N < 1, r < 0 or not finite, opts out of range, ... */
    JAC_ENOMEM = -2,   /* workspace too small, or host allocation failed */
    JAC_EDEVICE = -3,  /* a HIP call failed (message names it) */
    JAC_ENOCONV = -4,  /* max_sweeps reached without rho < tol */
    JAC_ENAN = -5      /* rho is NaN (a NaN or Inf reached the field, or R = ||b_A|| = 0: r = 0 with b = 0) */
};

/* Sweep kernels. */
enum jac_kernel {
    JAC_SYNC = 0,    /* (a) one synchronous sweep per launch */
    JAC_TBLOCK = 1,  /* (b) exact temporal blocking: D sweeps per launch, bitwise equal to (a) */
    JAC_ASYNC = 2,   /* (c) block-asynchronous: tile_x x tile_y tiles, frozen halo, D sweeps */
    JAC_SYNC_UNFUSED = 3  /* (a) without the fused right-hand side: each sweep reads u_k, u^n and s and
                             forms b = u^n + s per point (16 bytes per point per sweep instead of 12) --
                             the unfused baseline of page "stencil-jacobian.vercel.app", section 02 and
                             section 05 (Table VI); results identical to JAC_SYNC; LAUNCH and GRAPH only */
};

/* How a check's result reaches the decision (LAUNCH and GRAPH drivers; the
 * page's section 04, Table V: B = blocking, O = overlapped). */
enum jac_checks {
    JAC_CHECKS_OVERLAPPED = 0,  /* the residual of u_{gL} is fused into the first launch of the next
                                   interval, which is queued before the host reads check g; a launch
                                   that follows a stopping check returns at once.  A check that the
                                   step's last three checks extrapolate below 0.97 * tol runs as a
                                   residual pass alone; if it does not converge, the interval it
                                   skipped follows.  Results never depend on this.  Environment
                                   variable JACOBI_PREDICT_MARGIN=m at create time replaces 0.97
                                   (0 turns the prediction off).  TBLOCK with D >= 9 and D > M under
                                   LAUNCH: launches of up to D sweeps measure the residual of the
                                   levels where checks fall (at most two); a check that stops at an
                                   inner level is followed by a launch that recomputes that iterate
                                   from the launch's input; a launch ends on a predicted check.  Under
                                   LAUNCH, a TBLOCK check (and an ASYNC one in launches of at most 8
                                   sweeps whose tiles the one-lane strip kernel runs with a height
                                   that is a multiple of 8, such as 32 x 16) that is neither predicted
                                   to stop (below 1.25 * tol) nor within
                                   two intervals of the previous step's count measures the residual on
                                   every 8th row only, where no iterate can overflow: that maximum
                                   bounds R from below, so at or above tol it decides the check
                                   exactly; below tol the iterate is measured again in full.
                                   JACOBI_SAMPLED_CHECKS=n at create time sets the row stride (a power
                                   of two; 0 or 1: every row) */
    JAC_CHECKS_BLOCKING = 1     /* after each interval a standalone residual kernel, then the host waits
                                   for R and decides before anything more is queued */
};

/* Depth controllers for ASYNC (page "stencil-jacobian.vercel.app", section 02:
 * D is a launch argument and may change between launches).  They need the
 * LAUNCH driver; they imply JAC_CHECKS_BLOCKING.  G-asc and G-desc use the four
 * levels 1, 2, 4, 8 (three thresholds, four depths), each capped at opts.D:
 * the depth of a level L is min(L, opts.D), so with opts.D = 6 G-desc runs
 * 6, 4, 2, 1 and with opts.D = 16 neither exceeds 8.  Each time step starts
 * afresh. */
enum jac_controller {
    JAC_STATIC = 0,  /* D = opts.D throughout */
    JAC_G_ASC = 1,   /* start at 1; D steps up through 1, 2, 4, 8 (capped) as rho falls below 1e-2, 1e-3,
                        1e-4; latched (never steps back within a time step) */
    JAC_G_DESC = 2,  /* start at min(8, opts.D); D steps down through 8, 4, 2, 1 (capped) at the same
                        thresholds; latched */
    JAC_G_FB = 3     /* hill climbing on the measured convergence rate -ln(rho_g / rho_{g-1}) per ms:
                        start at 1; after each check (except the one right after a change, the
                        settling window) double D while the rate holds, halve it when the rate drops
                        by more than 10% against the previous measurement */
};

/* How the launches of a step are issued. */
enum jac_driver {
    JAC_LAUNCH = 0,      /* host enqueues each launch; reads each check back */
    JAC_GRAPH = 1,       /* each check interval captured once as a HIP graph and replayed */
    JAC_PERSISTENT = 2   /* one cooperative kernel per jac_solve: every step, check and decision on the
                            device; SYNC and TBLOCK use 2-D tiles in LDS with a D-cell ghost zone (held in
                            LDS for the whole solve when every tile fits one round of resident blocks,
                            re-staged per D sweeps otherwise), ASYNC its own tiles (held in LDS with a
                            one-cell halo under the same condition); same results as JAC_LAUNCH */
};

typedef struct {
    int32_t kernel;      /* jac_kernel */
    int32_t driver;      /* jac_driver */
    int32_t D;           /* sweeps per launch: TBLOCK 1..16, ASYNC 1..32; ignored for SYNC */
    int32_t tile_x;      /* ASYNC tile width in columns (1..256; tile_x * tile_y <= 4096; a check
                            takes one slot per block of the N*N/64 + 65536 in the workspace, so
                            jac_step / jac_solve reject, with JAC_EINVAL and before any work, tiles
                            whose launch needs more: only tiles under 64 points on large grids) */
    int32_t tile_y;      /* ASYNC tile height in rows (1..256) */
    int32_t M;           /* check interval in sweeps (>= 1).  SYNC and TBLOCK check every M sweeps
                            whatever D (a TBLOCK launch deeper than M measures the residual at the
                            levels where checks fall); ASYNC every max(M, D) */
    float tol;           /* rho threshold (> 0) */
    int32_t band_rows;   /* TBLOCK: rows per wavefront band (LAUNCH; for D >= 5 lowered where a band's rows
                            would span 2 GiB or more, which changes no result), tile side (PERSISTENT);
                            0: automatic */
    int64_t max_sweeps;  /* per step; a failed check at or past it ends with JAC_ENOCONV */
    int32_t checks;      /* jac_checks */
    int32_t controller;  /* jac_controller (ASYNC only) */
    int32_t overlap;     /* ASYNC: each tile iterates on itself widened by this many cells per side and
                            writes back only its own points -- overlapping subdomains (Islam & Wang,
                            "Hierarchical Jacobi Iteration ...", sections 3.5 and 4); 0..64 with
                            (tile_x + 2 overlap) * (tile_y + 2 overlap) <= 4096; LAUNCH and GRAPH only */
    int32_t reserved;    /* 0 */
} jac_opts;

/* SYNC, LAUNCH, D = 1, 32 x 8 tiles, M = 8, tol = 1e-5, band_rows = 0, max_sweeps = 1e6,
 * overlapped checks, static depth, no overlap (tol and M as page
 * "stencil-jacobian.vercel.app", section 01 fixes them; 32 x 8 blocks as its
 * section 02 names them). */
void jac_opts_default(jac_opts* opts);

/* Bytes of device workspace a context of size N needs: the two ping-pong
 * iterates, b and dt*f (the arrays of page "stencil-jacobian.vercel.app",
 * section 02, each padded with a ghost ring), plus scratch for the per-block
 * residual maxima, the persistent driver's barrier and its resident tiles'
 * edge exchange (at most 40 MiB).  0 if N is out of range (1..65536). */
size_t jac_workspace_bytes(int N);

/*
 * Create a context for an N x N grid with coupling r = alpha*dt/h^2 (>= 0)
 * (page "stencil-jacobian.vercel.app", section 01 "The problem": the N x N
 * grid of unknowns, the source f, boundary 100 on top and 0 elsewhere; the
 * coupling r is the one whose values 1, 10 and 100 set the sweeps per step).
 *   source_host  N*N floats, s = dt*f, copied during the call; NULL means 0.
 *   workspace    device memory of at least jac_workspace_bytes(N) bytes,
 *                256-byte aligned, owned by the caller, not freed by the
 *                library, and used by no one else while the context lives.
 *   stream       hipStream_t for every launch and copy (NULL: the null stream).
 * The field starts at u^0 = 0.  On success *out holds the context.
 */
int jac_create(int N, float r, const float* source_host, void* workspace, size_t ws_bytes,
               void* stream, jac_t* out);

/* One backward-Euler step (page "stencil-jacobian.vercel.app", section 01:
 * b = u^n + dt*f with u^n held fixed, then point Jacobi until rho < tol, tested
 * every M sweeps; section 02 for the kernels): on return the field is u^{n+1}
 * and *sweeps / *rho (either may be NULL) hold the sweep count and the rho of
 * the accepted iterate.  For SYNC and TBLOCK the result is bitwise identical to
 * the oracle's for the same M.  Blocks until the step's convergence is decided
 * (work the step queued ahead may still be draining on the stream).  Errors:
 * JAC_EINVAL for bad options (nothing is run), JAC_ENOCONV / JAC_ENAN (the field
 * is the last checked iterate), JAC_EDEVICE on a HIP failure. */
int jac_step(jac_t ctx, const jac_opts* opts, int64_t* sweeps, float* rho);

/* nsteps backward-Euler steps (page "stencil-jacobian.vercel.app", section 01:
 * ten steps, each starting from the previous step's converged field);
 * sweeps[n] and rho[n] for each (host arrays of nsteps, may be NULL).  Stops at
 * the first step that fails (ENOCONV / ENAN): the field is that step's last
 * checked iterate, later entries are 0 and NaN.  With JAC_PERSISTENT the whole
 * solve is one device kernel and the host waits once. */
int jac_solve(jac_t ctx, int nsteps, const jac_opts* opts, int64_t* sweeps, float* rho);

/* Throughput entry (the sweep kernels of page "stencil-jacobian.vercel.app",
 * section 02, without the convergence test of section 01): b = u^n + s, then
 * exactly nsweeps sweeps with no checks; the field is left at the last
 * iterate.  If rho != NULL it receives the rho of that iterate (one extra
 * residual pass).  Launches one by one whatever opts->driver says. */
int jac_sweep(jac_t ctx, const jac_opts* opts, int64_t nsweeps, float* rho);

/*
 * jac_sweep for callers that cannot allocate at call time (tight serving
 * loops, harnesses that forbid hipMalloc): the same launches and results as
 * jac_sweep, but the kernels' scratch -- the norm / check header and the
 * per-block partial maxima of the right-hand side and residual passes -- is
 * a static device array of the library (384 KiB, one copy per GPU, held until
 * the process ends) instead of the context's workspace, and the launch timer
 * is not used.  The call allocates no device or host memory and creates no
 * HIP object.  Limits: N <= 16384 and at most 32768 partial slots per launch;
 * beyond them JAC_EINVAL, nothing is run.  All calls on one GPU share the
 * array and each leaves its contents behind; every call re-initialises what it
 * reads before reading it, but calls that overlap in time on one GPU (two
 * streams, two threads) race on it and must not.  The call synchronizes the
 * context's stream, so it cannot be captured into a graph.  JAC_EDEVICE if the
 * device address of the array could not be found at jac_create.
 */
int jac_sweep_static(jac_t ctx, const jac_opts* opts, int64_t nsweeps, float* rho);

/* Copy the current field u^n to / from host memory (N*N floats, row-major,
 * row 0 next to the 100 boundary; the unknowns of page
 * "stencil-jacobian.vercel.app", section 01), for checkpoint and resume.
 * Blocking: waits for the context's stream.  Both enqueue on that stream one
 * 1-D copy of the N*N block through the idle iterate plane of the workspace
 * (the one the next sweep overwrites), a pitch-changing kernel and a refill of
 * that plane.  The host array is read (written) only during the call.
 * jac_set_field also resets the bound the constant-divisor division path
 * relies on (see below). */
int jac_get_field(jac_t ctx, float* host_out);
int jac_set_field(jac_t ctx, const float* host_in);

/* Set the field back to u^0 = 0 (device-side fill, no host traffic). */
int jac_reset(jac_t ctx);

/*
 * Division by d = 1 + 4r in the sweep.  The fast path multiplies by the
 * correctly rounded reciprocal and applies one fma correction; it has no
 * special-case fixup and differs from IEEE division only on numerators that
 * are Inf, NaN or -0.  jac_create enables it only after checking on the device
 * that it returns the IEEE quotient bit for bit on every other float input for
 * this d; environment variable JACOBI_IEEE_DIVISION=1 at create time disables
 * it.  Even then, each step (each jac_sweep, each persistent solve) uses it
 * only if the host can show that no such numerator occurs: the source holds no
 * -0, Inf or NaN, and a bound on |u| carried from step to step (a weighted-mean
 * bound, reset by jac_reset and jac_set_field) keeps every numerator finite;
 * otherwise that work divides by IEEE division.  Results are identical either
 * way.  Returns 1 if the fast path is enabled for the context, 0 if not,
 * < 0 on error.
 */
int jac_fast_division(jac_t ctx);

/* Division path the most recent step, sweep or persistent solve took: 1 the
 * fast path, 0 IEEE division (also before any work), < 0 on error. */
int jac_last_division(jac_t ctx);

/*
 * Depth of every check interval of the most recent jac_step / jac_solve call
 * (LAUNCH and GRAPH drivers; for SYNC the depth is 1), in order across its
 * steps: depths[i] for i < min(*count, cap); *count receives the number of
 * intervals.  With a depth controller this is the schedule it chose.
 */
int jac_depth_log(jac_t ctx, int32_t* depths, int64_t cap, int64_t* count);

/* Release the context (not the workspace).  NULL is accepted. */
int jac_destroy(jac_t ctx);

/* Message of the last failure on this thread ("" if none). */
const char* jac_last_error(void);

/*
 * Bandwidth probe (measurement only, no context needed; the analogue of the
 * bw_probe of page "cuda-solver-lab", section "Hardware ceilings"): on `stream`,
 * kind 0 copies a to c, kind 1 writes c = a + b (two reads, one write per
 * element, the traffic mix of a sweep); n floats, a multiple of 4, arrays
 * 16-byte aligned device memory owned by the caller; `blocks` workgroups of
 * 256 threads stride over the arrays; nontemporal != 0 marks the stores
 * nontemporal.  Asynchronous: time it with events on the stream.
 */
int jac_stream_probe(float* c, const float* a, const float* b, size_t n, int kind, int nontemporal,
                     int blocks, void* stream);

/*
 * Launch timing.  jac_profile(ctx, k) with k > 0 counts every kernel launch of
 * the library by class and brackets every k-th launch of each class with a
 * pair of HIP events on the context's stream (each event holds the next
 * kernel back by a few microseconds, so k = 1 slows small kernels noticeably);
 * k = 0 turns it off.
 * Enabling resets the counters.  jac_profile_read returns, for one class, the
 * summed device time of the bracketed launches, the number of launches and
 * the number bracketed.  Classes: 0 right-hand side, 1 sync sweep, 2 sync
 * sweep with check, 3 temporal-blocking launch, 4 block-async launch,
 * 5 residual only, 6 persistent solve, 7 launches issued ahead of a check that
 * stopped the step (they return at once and do no sweep), 8 one-block
 * reductions of a check or of ||b_A||, 9 the first temporal-blocking launch of
 * a step when it also forms b (launch driver, overlapped checks), 10 a deep
 * temporal-blocking launch shorter than D (one that ends on a check, or one
 * that recomputes the iterate a check inside a launch stopped at).
 */
int jac_profile(jac_t ctx, int every);
int jac_profile_read(jac_t ctx, int kclass, double* ms_timed, int64_t* launches, int64_t* timed_launches);

#ifdef __cplusplus
}
#endif
#endif /* LIBJACOBI_H */
