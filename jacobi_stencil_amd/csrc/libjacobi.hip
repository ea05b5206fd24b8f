// libjacobi.hip -- the C interface of include/jacobi.h and the host driver
// that issues a time step's launches.
//
// A step (page "stencil-jacobian.vercel.app", sections 01-02): form
// b = u^n + dt*f and ||b_A|| once, then sweep and test rho every L sweeps
// (L = M, or D when a launch does more than M sweeps) until rho < tol.
//
// How the host keeps the GPU busy across checks: the launches covering sweeps
// gL+1 .. (g+1)L form "group g".  The first launch of group g >= 1 also
// measures the residual of u_{gL} (the iterate it reads), so a check costs no
// extra pass over memory; the last block of that launch writes R to pinned
// host memory and, if the step must stop, sets a device flag that turns every
// later launch of the step into an immediate return.  The host enqueues group
// g+1 before it waits for check g, so the device never idles during the round
// trip, and a stop at check g leaves u_{gL} untouched in the buffer group g
// read from (its first launch wrote only the other buffer).
#include "../../include/jacobi.h"
#include "jacobi_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

using namespace jac;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

#define JAC_HIP(call)                                                                    \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess)                                                            \
            return fail(JAC_EDEVICE, std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

constexpr int kMaxN = 65536;
constexpr int kMaxD = 32;
constexpr int kClasses = 8;

enum KClass {
    KC_RHS = 0, KC_SYNC = 1, KC_SYNC_CHECK = 2, KC_TBLOCK = 3, KC_ASYNC = 4, KC_RESID = 5, KC_PERSIST = 6,
    KC_NOOP = 7  // launches issued ahead of a check that then stopped the step: they return at once
};

struct Pending {
    hipEvent_t e0, e1;
    int cls;
    int64_t group;  // check group within the step, -1 outside a step's sweep loop
    bool first;     // first launch of its group (the one that carries the check)
};

}  // namespace

struct jac_ctx {
    int N;
    float r, d;
    Geom g;
    hipStream_t stream;
    float* u[2];
    float* b;
    float* s;
    Scratch* sc;
    Mailbox* mail;   // pinned host memory written by the device
    int cur;         // u[cur] holds u^n
    hipEvent_t ev[kRing];
    int start_buf[kRing];
    // launch timing
    bool prof;
    std::vector<hipEvent_t> free_ev;
    std::vector<Pending> pending;
    int64_t cur_group;   // group being enqueued (tags profile entries)
    bool cur_first;
    double ms[kClasses];
    int64_t cnt[kClasses];
};

namespace {

StepArgs base_args(const jac_ctx* c, float tol) {
    StepArgs a;
    a.g = c->g;
    a.r = c->r;
    a.d = c->d;
    a.tol = tol;
    a.sc = c->sc;
    a.mail = c->mail;
    a.slot = 0;
    return a;
}

// Fold finished timing pairs into the per-class totals.  Entries of groups
// >= keep_from are left pending (their class may still change to KC_NOOP).
int drain_profile(jac_ctx* c, int64_t keep_from = INT64_MAX) {
    size_t w = 0;
    for (size_t i = 0; i < c->pending.size(); ++i) {
        Pending& p = c->pending[i];
        if (p.group >= keep_from) {
            c->pending[w++] = p;
            continue;
        }
        float ms = 0.0f;
        JAC_HIP(hipEventSynchronize(p.e1));
        JAC_HIP(hipEventElapsedTime(&ms, p.e0, p.e1));
        c->ms[p.cls] += ms;
        c->cnt[p.cls] += 1;
        c->free_ev.push_back(p.e0);
        c->free_ev.push_back(p.e1);
    }
    c->pending.resize(w);
    return JAC_OK;
}

// A stop at check group gs: every launch after the first of group gs returned
// at once; re-class them so they do not count as sweeps.
void mark_noops(jac_ctx* c, int64_t gs) {
    for (Pending& p : c->pending)
        if (p.group > gs || (p.group == gs && !p.first)) p.cls = KC_NOOP;
}

int take_event(jac_ctx* c, hipEvent_t* e) {
    if (c->free_ev.empty()) {
        JAC_HIP(hipEventCreate(e));
        return JAC_OK;
    }
    *e = c->free_ev.back();
    c->free_ev.pop_back();
    return JAC_OK;
}

// Run `fn` (which enqueues one kernel) bracketed by timing events when
// profiling is on.
template <class F>
int timed(jac_ctx* c, int cls, F&& fn) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (c->prof) {
        int st = take_event(c, &e0);
        if (st) return st;
        st = take_event(c, &e1);
        if (st) return st;
        JAC_HIP(hipEventRecord(e0, c->stream));
    }
    hipError_t e = fn();
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("kernel launch: ") + hipGetErrorString(e));
    if (c->prof) {
        JAC_HIP(hipEventRecord(e1, c->stream));
        c->pending.push_back({e0, e1, cls, c->cur_group, c->cur_first});
        c->cur_first = false;
    }
    return JAC_OK;
}

int check_opts(const jac_ctx* c, const jac_opts* o) {
    if (!o) return fail(JAC_EINVAL, "opts is NULL");
    if (o->kernel != JAC_SYNC && o->kernel != JAC_TBLOCK && o->kernel != JAC_ASYNC)
        return fail(JAC_EINVAL, "unknown kernel");
    if (o->driver != JAC_LAUNCH && o->driver != JAC_GRAPH && o->driver != JAC_PERSISTENT)
        return fail(JAC_EINVAL, "unknown driver");
    if (o->M < 1) return fail(JAC_EINVAL, "M must be >= 1");
    if (!(o->tol > 0.0f) || !std::isfinite(o->tol)) return fail(JAC_EINVAL, "tol must be a positive finite float");
    if (o->max_sweeps < 1) return fail(JAC_EINVAL, "max_sweeps must be >= 1");
    if (o->reserved != 0) return fail(JAC_EINVAL, "reserved must be 0");
    if (o->kernel != JAC_SYNC && (o->D < 1 || o->D > kMaxD)) return fail(JAC_EINVAL, "D must be in 1..32");
    if (o->kernel == JAC_ASYNC && (o->tile_x < 1 || o->tile_x > 256 || o->tile_y < 1 || o->tile_y > 256))
        return fail(JAC_EINVAL, "tile_x and tile_y must be in 1..256");
    if (o->kernel != JAC_SYNC) return fail(JAC_EINVAL, "this kernel is not available in this build");
    if (o->driver != JAC_LAUNCH) return fail(JAC_EINVAL, "this driver is not available in this build");
    (void)c;
    return JAC_OK;
}

// Sweeps per launch and the check interval for these options.
int sweeps_per_launch(const jac_opts* o) { return o->kernel == JAC_SYNC ? 1 : o->D; }
int64_t check_interval(const jac_opts* o) {
    int spl = sweeps_per_launch(o);
    return spl > o->M ? spl : o->M;
}

// Enqueue one launch of `m` sweeps from u[*buf] into the other buffer; with
// `check` it also measures the residual of its input into mailbox slot `slot`.
int enqueue_launch(jac_ctx* c, const jac_opts* o, int m, bool check, int slot, int* buf) {
    StepArgs a = base_args(c, o->tol);
    a.slot = slot;
    const float* in = c->u[*buf];
    float* out = c->u[*buf ^ 1];
    int st = JAC_OK;
    switch (o->kernel) {
        case JAC_SYNC:
            (void)m;
            st = timed(c, check ? KC_SYNC_CHECK : KC_SYNC,
                       [&] { return launch_sync(in, c->b, out, check, a, c->stream); });
            break;
        default:
            return fail(JAC_EINVAL, "kernel not available");
    }
    if (st) return st;
    *buf ^= 1;
    return JAC_OK;
}

// Enqueue the launches of sweeps [first, first + count) of a group.
int enqueue_sweeps(jac_ctx* c, const jac_opts* o, int64_t count, bool check_first, int slot, int* buf) {
    const int spl = sweeps_per_launch(o);
    bool check = check_first;
    while (count > 0) {
        int m = count < spl ? (int)count : spl;
        int st = enqueue_launch(c, o, m, check, slot, buf);
        if (st) return st;
        check = false;
        count -= m;
    }
    return JAC_OK;
}

int enqueue_rhs(jac_ctx* c, float tol) {
    StepArgs a = base_args(c, tol);
    return timed(c, KC_RHS, [&] { return launch_rhs(c->u[c->cur], c->s, c->b, a, c->stream); });
}

uint32_t read_mail(const volatile uint32_t* p) { return *p; }

int run_step(jac_ctx* c, const jac_opts* o, int64_t* sweeps_out, float* rho_out) {
    const int64_t L = check_interval(o);
    c->cur_group = -1;
    c->cur_first = false;
    int st = enqueue_rhs(c, o->tol);
    if (st) return st;
    int buf = c->cur;
    c->cur_group = 0;
    c->cur_first = true;
    st = enqueue_sweeps(c, o, L, false, 0, &buf);   // group 0: sweeps 1..L
    if (st) return st;

    int64_t g_enq = 1;          // next group to enqueue
    bool final_enqueued = false;
    auto enqueue_group = [&]() -> int {
        const int slot = (int)(g_enq % kRing);
        c->start_buf[slot] = buf;
        c->mail->R[slot] = kEmpty;
        StepArgs a = base_args(c, o->tol);
        a.slot = slot;
        c->cur_group = g_enq;
        c->cur_first = true;
        int s2;
        if (g_enq * L >= o->max_sweeps) {
            // the last allowed check: measure only, keep u_{gL} in place
            const float* in = c->u[buf];
            s2 = timed(c, KC_RESID, [&] { return launch_residual(in, c->b, a, c->stream); });
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[slot], c->stream));
            final_enqueued = true;
        } else {
            // one launch that checks u_{gL} and starts the next interval, then the rest
            const int64_t first = std::min<int64_t>(L, sweeps_per_launch(o));
            s2 = enqueue_sweeps(c, o, first, true, slot, &buf);
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[slot], c->stream));
            s2 = enqueue_sweeps(c, o, L - first, false, slot, &buf);
            if (s2) return s2;
        }
        ++g_enq;
        return JAC_OK;
    };

    st = enqueue_group();
    if (st) return st;
    for (int64_t g = 1;; ++g) {
        if (!final_enqueued && g_enq <= g + 1) {
            st = enqueue_group();
            if (st) return st;
        }
        const int slot = (int)(g % kRing);
        JAC_HIP(hipEventSynchronize(c->ev[slot]));
        const uint32_t Rb = read_mail(&c->mail->R[slot]);
        if (Rb == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
        float R, bAv;
        const uint32_t bAb = read_mail(&c->mail->bA_bits);
        std::memcpy(&R, &Rb, 4);
        std::memcpy(&bAv, &bAb, 4);
        const float rho = R / bAv;
        const int64_t k = g * L;
        const bool stop = !(rho >= o->tol);
        if (stop || k >= o->max_sweeps) {
            if (c->prof && stop) mark_noops(c, g);
            c->cur = c->start_buf[slot];
            if (sweeps_out) *sweeps_out = k;
            if (rho_out) *rho_out = rho;
            if (std::isnan(rho)) return fail(JAC_ENAN, "rho is NaN");
            if (!stop) return fail(JAC_ENOCONV, "max_sweeps reached before rho < tol");
            return JAC_OK;
        }
        if (c->prof && c->pending.size() > 8192) {
            st = drain_profile(c, g);  // groups before g are decided and finished
            if (st) return st;
        }
    }
}

}  // namespace

// ============================================================== C interface

extern "C" {

void jac_opts_default(jac_opts* o) {
    if (!o) return;
    o->kernel = JAC_SYNC;
    o->driver = JAC_LAUNCH;
    o->D = 1;
    o->tile_x = 32;
    o->tile_y = 8;
    o->M = 8;
    o->tol = 1e-5f;
    o->reserved = 0;
    o->max_sweeps = 1000000;
}

size_t jac_workspace_bytes(int N) {
    if (N < 1 || N > kMaxN) return 0;
    Geom g = make_geom(N);
    return (size_t)g.plane * 4 * sizeof(float) + sizeof(Scratch);
}

const char* jac_last_error(void) { return g_err.c_str(); }

int jac_create(int N, float r, const float* source_host, void* workspace, size_t ws_bytes, void* stream,
               jac_t* out) {
    if (!out) return fail(JAC_EINVAL, "out is NULL");
    *out = nullptr;
    if (N < 1 || N > kMaxN) return fail(JAC_EINVAL, "N must be in 1..65536");
    if (!(r >= 0.0f) || !std::isfinite(r)) return fail(JAC_EINVAL, "r must be finite and >= 0");
    if (!workspace) return fail(JAC_EINVAL, "workspace is NULL");
    if (((uintptr_t)workspace & 255u) != 0) return fail(JAC_EINVAL, "workspace must be 256-byte aligned");
    if (ws_bytes < jac_workspace_bytes(N)) return fail(JAC_ENOMEM, "workspace smaller than jac_workspace_bytes(N)");

    int dev = 0;
    JAC_HIP(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    JAC_HIP(hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(JAC_EDEVICE, std::string("libjacobi is built for gfx950; device is ") + prop.gcnArchName);

    jac_ctx* c = new (std::nothrow) jac_ctx();
    if (!c) return fail(JAC_ENOMEM, "host allocation failed");
    c->N = N;
    c->r = r;
    {
        float four_r = 4.0f * r;
        c->d = 1.0f + four_r;
    }
    c->g = make_geom(N);
    c->stream = (hipStream_t)stream;
    float* base = (float*)workspace;
    c->u[0] = base;
    c->u[1] = base + c->g.plane;
    c->b = base + 2 * c->g.plane;
    c->s = base + 3 * c->g.plane;
    c->sc = (Scratch*)(base + 4 * c->g.plane);
    c->cur = 0;
    c->prof = false;
    c->cur_group = -1;
    c->cur_first = false;
    for (int i = 0; i < kClasses; ++i) { c->ms[i] = 0.0; c->cnt[i] = 0; }
    for (int i = 0; i < kRing; ++i) c->ev[i] = nullptr;
    c->mail = nullptr;

    auto cleanup_fail = [&](int code) {
        jac_destroy(c);
        return code;
    };
    if (hipHostMalloc((void**)&c->mail, sizeof(Mailbox), hipHostMallocDefault) != hipSuccess)
        return cleanup_fail(fail(JAC_ENOMEM, "hipHostMalloc of the result mailbox failed"));
    std::memset(c->mail, 0xFF, sizeof(Mailbox));
    for (int i = 0; i < kRing; ++i)
        if (hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming) != hipSuccess)
            return cleanup_fail(fail(JAC_EDEVICE, "hipEventCreateWithFlags failed"));

    hipError_t e = launch_fill(base, c->g.plane * 4 + (int64_t)(sizeof(Scratch) / 4), 0.0f, c->stream);
    if (e == hipSuccess) e = launch_ghosts(c->u[0], c->g, c->stream);
    if (e == hipSuccess) e = launch_ghosts(c->u[1], c->g, c->stream);
    if (e == hipSuccess && source_host)
        e = hipMemcpy2DAsync(c->s + c->g.origin, (size_t)c->g.P * 4, source_host, (size_t)N * 4, (size_t)N * 4,
                             (size_t)N, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return cleanup_fail(fail(JAC_EDEVICE, std::string("set-up: ") + hipGetErrorString(e)));
    *out = c;
    return JAC_OK;
}

int jac_destroy(jac_t c) {
    if (!c) return JAC_OK;
    (void)hipStreamSynchronize(c->stream);
    for (int i = 0; i < kRing; ++i)
        if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
    for (Pending& p : c->pending) {
        (void)hipEventDestroy(p.e0);
        (void)hipEventDestroy(p.e1);
    }
    for (hipEvent_t e : c->free_ev) (void)hipEventDestroy(e);
    if (c->mail) (void)hipHostFree(c->mail);
    delete c;
    return JAC_OK;
}

int jac_step(jac_t c, const jac_opts* o, int64_t* sweeps, float* rho) { return jac_solve(c, 1, o, sweeps, rho); }

int jac_solve(jac_t c, int nsteps, const jac_opts* o, int64_t* sweeps, float* rho) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (nsteps < 0) return fail(JAC_EINVAL, "nsteps must be >= 0");
    int st = check_opts(c, o);
    if (st) return st;
    for (int n = 0; n < nsteps; ++n) {
        if (sweeps) sweeps[n] = 0;
        if (rho) rho[n] = NAN;
    }
    for (int n = 0; n < nsteps; ++n) {
        st = run_step(c, o, sweeps ? &sweeps[n] : nullptr, rho ? &rho[n] : nullptr);
        if (st) break;
    }
    if (c->prof) {
        int s2 = drain_profile(c);
        if (!st) st = s2;
    }
    return st;
}

int jac_sweep(jac_t c, const jac_opts* o, int64_t nsweeps, float* rho) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (nsweeps < 0) return fail(JAC_EINVAL, "nsweeps must be >= 0");
    int st = check_opts(c, o);
    if (st) return st;
    st = enqueue_rhs(c, o->tol);
    if (st) return st;
    int buf = c->cur;
    st = enqueue_sweeps(c, o, nsweeps, false, 0, &buf);
    if (st) return st;
    c->cur = buf;
    if (rho) {
        c->mail->R[0] = kEmpty;
        StepArgs a = base_args(c, o->tol);
        a.slot = 0;
        st = timed(c, KC_RESID, [&] { return launch_residual(c->u[c->cur], c->b, a, c->stream); });
        if (st) return st;
    }
    JAC_HIP(hipStreamSynchronize(c->stream));
    if (rho) {
        uint32_t Rb = read_mail(&c->mail->R[0]), bAb = read_mail(&c->mail->bA_bits);
        if (Rb == kEmpty) return fail(JAC_EDEVICE, "the residual did not report");
        float R, bAv;
        std::memcpy(&R, &Rb, 4);
        std::memcpy(&bAv, &bAb, 4);
        *rho = R / bAv;
    }
    if (c->prof) return drain_profile(c);
    return JAC_OK;
}

int jac_get_field(jac_t c, float* host_out) {
    if (!c || !host_out) return fail(JAC_EINVAL, "NULL argument");
    JAC_HIP(hipMemcpy2DAsync(host_out, (size_t)c->N * 4, c->u[c->cur] + c->g.origin, (size_t)c->g.P * 4,
                             (size_t)c->N * 4, (size_t)c->N, hipMemcpyDeviceToHost, c->stream));
    JAC_HIP(hipStreamSynchronize(c->stream));
    return JAC_OK;
}

int jac_set_field(jac_t c, const float* host_in) {
    if (!c || !host_in) return fail(JAC_EINVAL, "NULL argument");
    JAC_HIP(hipMemcpy2DAsync(c->u[c->cur] + c->g.origin, (size_t)c->g.P * 4, host_in, (size_t)c->N * 4,
                             (size_t)c->N * 4, (size_t)c->N, hipMemcpyHostToDevice, c->stream));
    JAC_HIP(hipStreamSynchronize(c->stream));
    return JAC_OK;
}

int jac_reset(jac_t c) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    JAC_HIP(launch_fill(c->u[0], c->g.plane * 2, 0.0f, c->stream));
    JAC_HIP(launch_ghosts(c->u[0], c->g, c->stream));
    JAC_HIP(launch_ghosts(c->u[1], c->g, c->stream));
    c->cur = 0;
    JAC_HIP(hipStreamSynchronize(c->stream));
    return JAC_OK;
}

int jac_profile(jac_t c, int enable) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (c->prof) {
        int st = drain_profile(c);
        if (st) return st;
    }
    c->prof = enable != 0;
    for (int i = 0; i < kClasses; ++i) { c->ms[i] = 0.0; c->cnt[i] = 0; }
    return JAC_OK;
}

int jac_profile_read(jac_t c, int kclass, double* ms_total, int64_t* launches) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (kclass < 0 || kclass >= kClasses) return fail(JAC_EINVAL, "unknown kernel class");
    int st = drain_profile(c);
    if (st) return st;
    if (ms_total) *ms_total = c->ms[kclass];
    if (launches) *launches = c->cnt[kclass];
    return JAC_OK;
}

}  // extern "C"
