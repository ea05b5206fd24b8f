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
// extra pass over memory; a one-block reduction that follows it writes R to
// the coherent host mailbox and, if the step must stop, sets a device flag
// that turns every later launch of the step into an immediate return.  The host enqueues group
// g+1 before it waits for check g, so the device never idles during the round
// trip, and a stop at check g leaves u_{gL} untouched in the buffer group g
// read from (its first launch wrote only the other buffer).
#include "../../include/jacobi.h"
#include "jacobi_internal.h"
#include "check_predict.h"

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <chrono>
#include <thread>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

using namespace jac;

namespace jac {
// kernels_async.hip: whether checking launches of D sweeps on this tiling
// honour a row mask of 7 (take a check's residual on every 8th row)
bool async_samples_rows(int N, int tx, int ty, int o, int D);
// kernels_copy.hip: an N x N block from pitch spitch to pitch dpitch
hipError_t launch_copy_rect(float* dst, int64_t dpitch, const float* src, int64_t spitch, int N, hipStream_t s);
}  // namespace jac

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
constexpr int kMaxTBlockD = 16;
constexpr int kClasses = 11;

enum KClass {
    KC_RHS = 0, KC_SYNC = 1, KC_SYNC_CHECK = 2, KC_TBLOCK = 3, KC_ASYNC = 4, KC_RESID = 5, KC_PERSIST = 6,
    KC_NOOP = 7,   // launches issued ahead of a check that then stopped the step: they return at once
    KC_REDUCE = 8,  // one-block reductions of a check's or a norm's partial maxima
    KC_TBLOCK_RHS = 9,  // a step's first temporal-blocking launch, which also forms b
    KC_TBLOCK_PART = 10  // deep temporal blocking: a launch shorter than D (ends on a check, or a redo)
};

// One launch as seen by the launch timer.
struct Rec {
    int cls;
    int64_t step;    // serial of the step it belongs to
    int64_t group;   // check group within the step, -1 outside the sweep loop
    bool first;      // first launch of its group (the one that carries the check)
    hipEvent_t e0, e1;  // timing pair when this launch was sampled, else null
};

// ---- static scratch for jac_sweep_static (an entry point that allocates nothing)
//
// The scratch header, the (unused) barrier-flag lines and kStaticPartials
// per-block partial maxima, laid out as in a workspace's scratch region.  Each
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, once per device (static_scratch_on).
constexpr int64_t kStaticPartials = 32768;
constexpr int kStaticMaxN = 16384;
constexpr size_t kStaticScratchBytes =
    sizeof(Scratch) + (size_t)kMaxPersistBlocks * kFlagStride * 4 + (size_t)kStaticPartials * 4;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_static_mu;
Scratch* g_static_sc[kMaxDevices];      // device address of `scratch` on each device (null: none)
hipError_t g_static_err[kMaxDevices];  // why a device's lookup failed (hipSuccess: not failed)

}  // namespace

struct jac_ctx {
    int N;
    float r, d, y;
    int fastdiv;     // 1: the constant-divisor quotient was verified for this d
    bool rhs_pending;  // the next temporal-blocking launch forms b itself (first of a step)
    float predict_margin;  // overlapped checks: a check predicted below margin * tol runs alone (0: never)
    int sample_rows;       // deep temporal blocking: checks far from the stop measure every sample_rows-th row (0: off)
    int64_t prev_sweeps;   // sweeps of the previous step (0: none yet)
    int64_t verified;      // sampled checks below tol measured again in full
    int cur_smask;         // row mask of the next checking temporal-blocking launch (0: every row)
    int fast_now;    // division path of the work being enqueued (see division_path)
    bool src_plain;  // the source is finite and holds no -0
    double smax;     // max |s|
    double ubound;   // upper bound on max |u| over u^n and its ghost ring (Inf: none)
    int graph_fast;  // division path the cached graphs were captured with
    std::vector<int32_t> dlog;  // depth of each check interval of the last jac_solve
    int cus;         // compute units of the device
    void* pout;      // pinned records of the persistent driver
    int pout_cap;
    // graph driver: one captured check interval per start buffer, for the
    // options they were captured with
    hipStream_t cap_stream;
    bool graphs_valid;
    jac_opts graph_key;
    hipGraphExec_t g_first[2];  // sweeps 1..L of a step (no check), by start buffer
    hipGraphExec_t g_group[2];  // one checking interval, by start buffer
    int g_flips_first, g_flips_group;  // buffer parity change across each graph
    int tb_rows[kMaxTBlockD + 1];  // automatic band height per depth (0: not yet computed)
    int sync_rows;                 // rows per wavefront of the synchronous sweep
    Geom g;
    hipStream_t stream;
    float* u[2];
    float* b;
    float* s;
    Scratch* sc;
    int64_t npart_cap;
    uint64_t* xchg;          // edge exchange of the persistent kernel's resident tiles
    Scratch* static_sc;      // this device's copy of the static scratch array (jac_sweep_static)
    hipError_t static_err;   // why it is missing, if it is
    Mailbox* mail;   // pinned host memory written by the device
    int cur;         // u[cur] holds u^n
    hipEvent_t ev[kRing];
    int start_buf[kRing];
    // launch timing
    int prof_every;  // 0: off; k: time every k-th launch of each class
    std::vector<hipEvent_t> free_ev;
    std::vector<Rec> recs;
    int64_t step_serial;
    int64_t cur_group;
    bool cur_first;
    int64_t seen[kClasses];
    double ms[kClasses];
    int64_t cnt[kClasses];
    int64_t timed_n[kClasses];
};

namespace {

// Division path for the next piece of work: `steps` rounds of (b = u + s,
// then at most `sweeps` sweeps).  The fast quotient is exact on every float
// numerator except Inf, NaN and -0, so it is taken only where none can occur.
// -0: n = b + r*S is -0 only if b is (a rounded sum is -0 only when both
// terms are), and b = u + s only if s is -- the source has none.  Inf/NaN:
// each update is a weighted mean, u' = (b + r*(uE+uW+uN+uS)) / (1 + 4r), so
// with U bounding |u| and B = U + max|s| bounding |b|, |u| stays below
// max(U, B) = B up to at most 8 roundings per sweep, a factor below
// (1 + 2^-20) per sweep; then no intermediate of the update exceeds
// B' + 4r B', B' the grown bound, and if that is finite no numerator overflows.
// The bound only grows: it is refreshed from the sweeps actually run after
// each step, and reset by jac_reset / jac_set_field.
int division_path(const jac_ctx* c, int steps, double sweeps, double* u_after = nullptr) {
    if (!c->fastdiv || !c->src_plain) return 0;
    double U = c->ubound;
    const double grow = std::exp(sweeps * std::ldexp(1.0, -20));
    for (int n = 0; n < steps; ++n) {
        const double B = (U + c->smax) * grow;
        if (!((B + 4.0 * (double)c->r * B) * 1.001 < (double)FLT_MAX)) return 0;
        U = B;
    }
    if (u_after) *u_after = U;
    return 1;
}

// Refresh the bound after work that ran `sweeps` sweeps after one RHS.
void grow_ubound(jac_ctx* c, double sweeps) {
    c->ubound = (c->ubound + c->smax) * std::exp(sweeps * std::ldexp(1.0, -20));
}

StepArgs base_args(const jac_ctx* c, float tol) {
    StepArgs a;
    a.g = c->g;
    a.r = c->r;
    a.d = c->d;
    a.y = c->y;
    a.fastdiv = c->fast_now;
    a.tol = tol;
    a.sc = c->sc;
    a.mail = c->mail;
    a.slot = 0;
    a.chk[0] = 0;
    a.chk[1] = -1;
    a.force = 0;
    a.part_off = 0;
    a.slot2 = -1;
    a.smask[0] = 0;
    a.smask[1] = 0;
    return a;
}

// Fold the records of steps before `keep_step` into the per-class totals.
int drain_profile(jac_ctx* c, int64_t keep_step = INT64_MAX) {
    size_t w = 0;
    for (size_t i = 0; i < c->recs.size(); ++i) {
        Rec& p = c->recs[i];
        if (p.step >= keep_step) {
            c->recs[w++] = p;
            continue;
        }
        c->cnt[p.cls] += 1;
        if (p.e0) {
            float ms = 0.0f;
            JAC_HIP(hipEventSynchronize(p.e1));
            JAC_HIP(hipEventElapsedTime(&ms, p.e0, p.e1));
            c->ms[p.cls] += ms;
            c->timed_n[p.cls] += 1;
            c->free_ev.push_back(p.e0);
            c->free_ev.push_back(p.e1);
        }
    }
    c->recs.resize(w);
    return JAC_OK;
}

// A stop at check group gs of the current step: every sweep launch after the
// first of group gs returned at once; re-class them so they do not count.
void mark_noops(jac_ctx* c, int64_t gs) {
    for (Rec& p : c->recs)
        if (p.step == c->step_serial && p.cls != KC_REDUCE && (p.group > gs || (p.group == gs && !p.first)))
            p.cls = KC_NOOP;
}

// Timing events: no system-scope fence when recorded (they only time work).
int take_event(jac_ctx* c, hipEvent_t* e) {
    if (c->free_ev.empty()) {
        JAC_HIP(hipEventCreateWithFlags(e, hipEventDisableSystemFence));
        return JAC_OK;
    }
    *e = c->free_ev.back();
    c->free_ev.pop_back();
    return JAC_OK;
}

// Run `fn` (which enqueues one kernel) and, when the launch timer is on,
// record it -- bracketed by a pair of HIP events if it is sampled.  Events
// between launches cost ~10 us of dispatch gap each, so only every k-th launch
// of a class is bracketed.
template <class F>
int timed(jac_ctx* c, int cls, F&& fn) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool sample = c->prof_every > 0 && (c->seen[cls]++ % c->prof_every) == 0;
    if (sample) {
        int st = take_event(c, &e0);
        if (st) return st;
        st = take_event(c, &e1);
        if (st) return st;
        JAC_HIP(hipEventRecord(e0, c->stream));
    }
    hipError_t e = fn();
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("kernel launch: ") + hipGetErrorString(e));
    if (sample) JAC_HIP(hipEventRecord(e1, c->stream));
    if (c->prof_every > 0) c->recs.push_back({cls, c->step_serial, c->cur_group, c->cur_first, e0, e1});
    if (cls != KC_REDUCE) c->cur_first = false;
    return JAC_OK;
}

bool is_sync(const jac_opts* o) { return o->kernel == JAC_SYNC || o->kernel == JAC_SYNC_UNFUSED; }

int check_opts(const jac_ctx* c, const jac_opts* o) {
    if (!o) return fail(JAC_EINVAL, "opts is NULL");
    if (o->kernel != JAC_SYNC && o->kernel != JAC_TBLOCK && o->kernel != JAC_ASYNC && o->kernel != JAC_SYNC_UNFUSED)
        return fail(JAC_EINVAL, "unknown kernel");
    if (o->checks != JAC_CHECKS_OVERLAPPED && o->checks != JAC_CHECKS_BLOCKING)
        return fail(JAC_EINVAL, "unknown checks mode");
    if (o->controller < JAC_STATIC || o->controller > JAC_G_FB) return fail(JAC_EINVAL, "unknown controller");
    if (o->controller != JAC_STATIC && (o->kernel != JAC_ASYNC || o->driver != JAC_LAUNCH))
        return fail(JAC_EINVAL, "depth controllers need the ASYNC kernel and the LAUNCH driver");
    if (o->overlap != 0 && o->kernel != JAC_ASYNC) return fail(JAC_EINVAL, "overlap is an ASYNC option");
    if (o->overlap < 0 || o->overlap > 64) return fail(JAC_EINVAL, "overlap must be in 0..64");
    if (o->reserved != 0) return fail(JAC_EINVAL, "reserved must be 0");
    if (o->driver == JAC_PERSISTENT && (o->kernel == JAC_SYNC_UNFUSED || o->overlap != 0))
        return fail(JAC_EINVAL, "the persistent driver runs SYNC, TBLOCK and ASYNC without overlap");
    if (o->driver != JAC_LAUNCH && o->driver != JAC_GRAPH && o->driver != JAC_PERSISTENT)
        return fail(JAC_EINVAL, "unknown driver");
    if (o->M < 1) return fail(JAC_EINVAL, "M must be >= 1");
    if (!(o->tol > 0.0f) || !std::isfinite(o->tol)) return fail(JAC_EINVAL, "tol must be a positive finite float");
    if (o->max_sweeps < 1) return fail(JAC_EINVAL, "max_sweeps must be >= 1");
    if (o->band_rows < 0 || o->band_rows > 65536) return fail(JAC_EINVAL, "band_rows must be in 0..65536");
    if (!is_sync(o) && (o->D < 1 || o->D > kMaxD)) return fail(JAC_EINVAL, "D must be in 1..32");
    if (o->kernel == JAC_ASYNC && (o->tile_x < 1 || o->tile_x > 256 || o->tile_y < 1 || o->tile_y > 256 ||
                                   (int64_t)(o->tile_x + 2 * o->overlap) * (o->tile_y + 2 * o->overlap) > 4096))
        return fail(JAC_EINVAL,
                    "tile_x and tile_y must be in 1..256 with (tile_x + 2 overlap) * (tile_y + 2 overlap) <= 4096");
    if (o->kernel == JAC_TBLOCK && o->D > kMaxTBlockD) return fail(JAC_EINVAL, "TBLOCK needs D in 1..16");
    (void)c;
    return JAC_OK;
}

// Sweeps per launch and the check interval for these options.
int sweeps_per_launch(const jac_opts* o) { return is_sync(o) ? 1 : o->D; }
// Temporal blocking checks every M sweeps whatever D: a launch deeper than M
// measures the residual at the levels where checks fall (run_step_deep), and
// the other drivers launch at most M sweeps at a time.  The block-asynchronous
// kernel checks every max(M, D): its in-tile sweeps are not global iterates.
int64_t check_interval(const jac_opts* o) {
    if (o->kernel == JAC_TBLOCK) return o->M;
    int spl = sweeps_per_launch(o);
    return spl > o->M ? spl : o->M;
}

// Reduce the partial maxima a check launch of `npart` blocks wrote into
// mailbox slot `slot` (and the device stop flag).
int enqueue_check_reduce(jac_ctx* c, int64_t npart, float tol, int slot) {
    if (npart > c->npart_cap) return fail(JAC_EDEVICE, "launch exceeds the partial-maximum slots");
    StepArgs a = base_args(c, tol);
    a.slot = slot;
    return timed(c, KC_REDUCE, [&] { return launch_reduce(npart, false, a, c->stream); });
}

// Enqueue one launch of `m` sweeps from u[*buf] into the other buffer; with
// `check` it also measures the residual of its input and reduces it into
// mailbox slot `slot`.
int enqueue_launch(jac_ctx* c, const jac_opts* o, int m, bool check, int slot, int* buf) {
    StepArgs a = base_args(c, o->tol);
    a.slot = slot;
    const float* in = c->u[*buf];
    float* out = c->u[*buf ^ 1];
    int st = JAC_OK;
    int64_t npart = 0;
    switch (o->kernel) {
        case JAC_SYNC:
        case JAC_SYNC_UNFUSED: {
            (void)m;
            npart = sync_blocks(c->N, c->sync_rows);
            if (check && npart > c->npart_cap) return fail(JAC_EDEVICE, "sync grid exceeds partial slots");
            const float* src = o->kernel == JAC_SYNC_UNFUSED ? c->s : nullptr;
            st = timed(c, check ? KC_SYNC_CHECK : KC_SYNC,
                       [&] { return launch_sync(in, c->b, src, out, check, c->sync_rows, a, c->stream); });
            break;
        }
        case JAC_TBLOCK: {
            if (o->band_rows == 0 && c->tb_rows[m] == 0)
                c->tb_rows[m] = tblock_rows(c->N, m, c->cus, tblock_waves_per_cu(m, c->fastdiv != 0));
            const int Hmax = tblock_max_rows(c->N, m);  // any height gives the same bits
            const int H = std::min(o->band_rows > 0 ? o->band_rows : c->tb_rows[m], Hmax);
            npart = tblock_blocks(c->N, m, H);
            if (c->rhs_pending && !check) {
                // b = u^n + s formed in this launch, then ||b_A|| from its partial maxima
                c->rhs_pending = false;
                if (npart > c->npart_cap)
                    return fail(JAC_EINVAL, "band_rows too small for this N: too many wavefront bands");
                st = timed(c, KC_TBLOCK_RHS,
                           [&] { return launch_tblock_rhs(in, c->s, c->b, out, m, a, H, c->stream); });
                if (st) return st;
                st = timed(c, KC_REDUCE, [&] { return launch_reduce(npart, true, a, c->stream); });
                if (st) return st;
                *buf ^= 1;
                return JAC_OK;
            }
            if (check && npart > c->npart_cap)
                return fail(JAC_EINVAL, "band_rows too small for this N: too many wavefront bands");
            if (check) a.smask[0] = c->cur_smask;
            st = timed(c, KC_TBLOCK, [&] { return launch_tblock(in, c->b, out, m, check, a, H, c->stream); });
            break;
        }
        case JAC_ASYNC:
            npart = async_blocks(c->N, o->tile_x, o->tile_y, o->overlap);
            if (check && npart > c->npart_cap) return fail(JAC_EINVAL, "tile too small for this N");
            if (check) a.smask[0] = c->cur_smask;
            st = timed(c, KC_ASYNC, [&] {
                return launch_async(in, c->b, out, o->tile_x, o->tile_y, m, o->overlap, check, a, c->stream);
            });
            break;
        default:
            return fail(JAC_EINVAL, "kernel not available");
    }
    if (st) return st;
    if (check) {
        st = enqueue_check_reduce(c, npart, o->tol, slot);
        if (st) return st;
    }
    *buf ^= 1;
    return JAC_OK;
}

// Enqueue the launches of `count` sweeps; the first may carry a check.
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

// b = u^n + s and ||b_A|| (which also clears the stop flag).  For the
// unfused sweep the b plane keeps u^n instead.
int enqueue_rhs(jac_ctx* c, const jac_opts* o) {
    StepArgs a = base_args(c, o->tol);
    const int64_t npart = rhs_blocks(c->N);
    if (npart > c->npart_cap) return fail(JAC_EDEVICE, "rhs grid exceeds partial slots");
    const bool keep_u = o->kernel == JAC_SYNC_UNFUSED;
    int st = timed(c, KC_RHS, [&] { return launch_rhs(c->u[c->cur], c->s, c->b, keep_u, a, c->stream); });
    if (st) return st;
    return timed(c, KC_REDUCE, [&] { return launch_reduce(npart, true, a, c->stream); });
}

// The residual of u[buf] alone (no sweep), reduced into mailbox slot `slot`.
int enqueue_residual(jac_ctx* c, const jac_opts* o, int buf, int slot) {
    StepArgs a = base_args(c, o->tol);
    a.slot = slot;
    const float* in = c->u[buf];
    const float* src = o->kernel == JAC_SYNC_UNFUSED ? c->s : nullptr;
    int st = timed(c, KC_RESID, [&] { return launch_residual(in, c->b, src, c->sync_rows, a, c->stream); });
    if (st) return st;
    return enqueue_check_reduce(c, sync_blocks(c->N, c->sync_rows), o->tol, slot);
}

uint32_t read_mail(const volatile uint32_t* p) { return *p; }

// A check's R after its event: the reduction's store normally has landed when
// the event completes; if the slot still reads empty, poll it briefly, then
// wait for the whole stream and read it once more.
uint32_t await_mail(jac_ctx* c, const volatile uint32_t* p) {
    uint32_t v = *p;
    if (v != kEmpty) return v;
    const auto t0 = std::chrono::steady_clock::now();
    while ((v = *p) == kEmpty && std::chrono::steady_clock::now() - t0 < std::chrono::milliseconds(100))
        std::this_thread::yield();
    if (v != kEmpty) return v;
    (void)hipStreamSynchronize(c->stream);
    return *p;
}

float mail_float(const volatile uint32_t* p) {
    const uint32_t b = *p;
    float f;
    std::memcpy(&f, &b, 4);
    return f;
}

// ---- graph driver: capture one interval of launches, replay it

void drop_graphs(jac_ctx* c) {
    for (int i = 0; i < 2; ++i) {
        if (c->g_first[i]) (void)hipGraphExecDestroy(c->g_first[i]);
        if (c->g_group[i]) (void)hipGraphExecDestroy(c->g_group[i]);
        c->g_first[i] = c->g_group[i] = nullptr;
    }
    c->graphs_valid = false;
}

bool same_graph_key(const jac_opts* a, const jac_opts* b) {
    return a->kernel == b->kernel && a->D == b->D && a->M == b->M && a->tile_x == b->tile_x &&
           a->tile_y == b->tile_y && a->band_rows == b->band_rows && a->tol == b->tol && a->overlap == b->overlap;
}

// Capture the launches of one interval starting from u[start] on a private
// stream.  The checking launch's reduction takes its mailbox slot from the
// device's check counter, so the graph replays with constant arguments.
int capture_interval(jac_ctx* c, const jac_opts* o, int start, bool check, hipGraphExec_t* out, int* flips) {
    if (!c->cap_stream) JAC_HIP(hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
    const hipStream_t saved = c->stream;
    const int saved_prof = c->prof_every;
    c->stream = c->cap_stream;
    c->prof_every = 0;
    int st = JAC_OK;
    hipError_t e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
    int buf = start;
    if (e == hipSuccess) {
        const int64_t L = check_interval(o);
        if (check) {
            const int64_t first = std::min<int64_t>(L, sweeps_per_launch(o));
            st = enqueue_sweeps(c, o, first, true, -1, &buf);
            if (!st) st = enqueue_sweeps(c, o, L - first, false, -1, &buf);
        } else {
            st = enqueue_sweeps(c, o, L, false, -1, &buf);
        }
    }
    hipGraph_t graph = nullptr;
    if (e == hipSuccess) {
        hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
        if (e2 != hipSuccess && !st) st = fail(JAC_EDEVICE, std::string("hipStreamEndCapture: ") + hipGetErrorString(e2));
    }
    c->stream = saved;
    c->prof_every = saved_prof;
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
    if (st) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    e = hipGraphInstantiate(out, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    *flips = buf != start;
    return JAC_OK;
}

int graph_for(jac_ctx* c, const jac_opts* o, bool check, int start, hipGraphExec_t* g, int* flips) {
    if (!c->graphs_valid || !same_graph_key(&c->graph_key, o) || c->graph_fast != c->fast_now) {
        drop_graphs(c);
        c->graph_key = *o;
        c->graphs_valid = true;
        c->graph_fast = c->fast_now;
    }
    hipGraphExec_t* slot = check ? &c->g_group[start] : &c->g_first[start];
    int* fl = check ? &c->g_flips_group : &c->g_flips_first;
    if (!*slot) {
        int st = capture_interval(c, o, start, check, slot, fl);
        if (st) return st;
    }
    *g = *slot;
    *flips = *fl;
    return JAC_OK;
}

// ---- depth controllers (page "stencil-jacobian.vercel.app", section 02)

// G-asc / G-desc levels: the depth steps as rho crosses 1e-2, 1e-3, 1e-4,
// compared as binary32 values.
int asc_level(float rho) { return rho >= 1e-2f ? 1 : rho >= 1e-3f ? 2 : rho >= 1e-4f ? 4 : 8; }
int desc_level(float rho) { return rho >= 1e-2f ? 8 : rho >= 1e-3f ? 4 : rho >= 1e-4f ? 2 : 1; }

struct DepthControl {
    int kind, Dmax, D;
    float prev_rho;    // G-fb: rho of the previous check (NaN: none yet)
    double prev_rate;  // G-fb: the last rate compared against (NaN: none yet)
    int settle;        // G-fb: checks still to skip after a change

    // G-asc / G-desc take the levels 1, 2, 4, 8, each capped at Dmax.
    DepthControl(int k, int dmax) : kind(k), Dmax(dmax), D(dmax), prev_rho(NAN), prev_rate(NAN), settle(0) {
        if (kind == JAC_G_ASC || kind == JAC_G_FB) D = 1;
        if (kind == JAC_G_DESC) D = std::min(8, Dmax);
    }
    // After a check of an interval run at depth D that took `ms` milliseconds.
    void update(float rho, double ms) {
        if (kind == JAC_G_ASC) {
            D = std::max(D, std::min(asc_level(rho), Dmax));
        } else if (kind == JAC_G_DESC) {
            D = std::min(D, std::min(desc_level(rho), Dmax));
        } else if (kind == JAC_G_FB) {
            const float before = prev_rho;
            prev_rho = rho;
            if (std::isnan(before) || !(ms > 0.0)) return;
            const double rate = -std::log((double)rho / (double)before) / ms;
            if (settle > 0) {  // the residual bump right after a change
                --settle;
                return;
            }
            const bool drop = !std::isnan(prev_rate) && rate < 0.9 * prev_rate;
            prev_rate = rate;
            const int next = drop ? std::max(1, D / 2) : std::min(Dmax, D * 2);
            if (next != D) {
                D = next;
                settle = 1;
            }
        }
    }
};

// One step with blocking checks: after each interval a standalone residual
// kernel, then the host waits for R and decides -- and, under a depth
// controller, picks the next interval's depth -- before queueing more.
int run_step_blocking(jac_ctx* c, const jac_opts* o, int64_t* sweeps_out, float* rho_out) {
    const int64_t L = check_interval(o);
    const bool graph = o->driver == JAC_GRAPH;
    c->fast_now = division_path(c, 1, (double)o->max_sweeps + (double)L);
    c->step_serial += 1;
    c->cur_group = -1;
    c->cur_first = false;
    if (c->prof_every > 0) {
        int s0 = drain_profile(c, c->step_serial - 1);
        if (s0) return s0;
    }
    int st = enqueue_rhs(c, o);
    if (st) return st;
    int buf = c->cur;
    DepthControl ctl(o->controller, is_sync(o) ? 1 : o->D);
    jac_opts oi = *o;
    for (int64_t g = 1;; ++g) {
        oi.D = ctl.D;
        c->cur_group = g;
        c->cur_first = true;
        const auto t0 = std::chrono::steady_clock::now();
        if (graph) {
            hipGraphExec_t gx;
            int flips;
            st = graph_for(c, &oi, false, buf, &gx, &flips);
            if (st) return st;
            JAC_HIP(hipGraphLaunch(gx, c->stream));
            buf ^= flips;
        } else {
            st = enqueue_sweeps(c, &oi, L, false, 0, &buf);
            if (st) return st;
        }
        const int slot = (int)((g - 1) % kRing);
        c->mail->R[slot] = kEmpty;
        st = enqueue_residual(c, o, buf, slot);
        if (st) return st;
        const int ev = (int)(g % kRing);
        JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
        JAC_HIP(hipEventSynchronize(c->ev[ev]));
        const uint32_t Rb = await_mail(c, &c->mail->R[slot]);
        const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        if (Rb == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
        const float R = mail_float(&c->mail->R[slot]);
        const float rho = R / mail_float(&c->mail->bA_bits);
        c->dlog.push_back(oi.D);
        const int64_t k = g * L;
        const bool stop = !(rho >= o->tol);
        if (stop || k >= o->max_sweeps) {
            c->cur = buf;
            if (sweeps_out) *sweeps_out = k;
            if (rho_out) *rho_out = rho;
            if (std::isnan(rho)) return fail(JAC_ENAN, "rho is NaN");
            if (!stop) return fail(JAC_ENOCONV, "max_sweeps reached before rho < tol");
            return JAC_OK;
        }
        ctl.update(rho, ms);
        if (c->prof_every > 0 && c->recs.size() > 8192) {
            st = drain_profile(c, c->step_serial);
            if (st) return st;
        }
    }
}

// One temporal-blocking launch of m sweeps from u[*buf] into the other buffer
// for the deep driver.  levels[q] (q < 2; -1: none) are the launch's levels
// whose residual it measures, for checks g[q]: each is reduced into mailbox slot
// (g - 1) % kRing and followed by that check's event.  `force` runs it even
// after a check has stopped the step (a redo).
int enqueue_tb_deep(jac_ctx* c, const jac_opts* o, int m, const int* levels, const int64_t* g, bool force,
                    int* buf, const int* smask = nullptr) {
    StepArgs a = base_args(c, o->tol);
    const bool check = levels[0] >= 0;
    a.chk[0] = levels[0];
    a.chk[1] = levels[1];
    if (smask) {
        a.smask[0] = smask[0];
        a.smask[1] = smask[1];
    }
    a.force = force ? 1 : 0;
    a.slot = check ? (int)((g[0] - 1) % kRing) : 0;
    if (check && m <= 8 && (levels[0] != 0 || levels[1] >= 0))
        return fail(JAC_EDEVICE, "a launch of 8 sweeps or fewer checks only its input");
    if (o->band_rows == 0 && c->tb_rows[m] == 0)
        c->tb_rows[m] = tblock_rows(c->N, m, c->cus, tblock_waves_per_cu(m, c->fastdiv != 0));
    const int Hmax = tblock_max_rows(c->N, m);
    const int H = std::min(o->band_rows > 0 ? o->band_rows : c->tb_rows[m], Hmax);
    const int64_t npart = tblock_blocks(c->N, m, H);
    if (check && 2 * npart > c->npart_cap)
        return fail(JAC_EINVAL, "band_rows too small for this N: too many wavefront bands");
    const float* in = c->u[*buf];
    float* out = c->u[*buf ^ 1];
    int st = timed(c, m == o->D ? KC_TBLOCK : KC_TBLOCK_PART,
                   [&] { return launch_tblock(in, c->b, out, m, check, a, H, c->stream); });
    if (st) return st;
    if (check) {
        // one reduction for both checked levels: partial slots [0, npart) and [npart, 2 npart)
        StepArgs ra = base_args(c, o->tol);
        ra.slot = (int)((g[0] - 1) % kRing);
        ra.slot2 = levels[1] >= 0 ? (int)((g[1] - 1) % kRing) : -1;
        st = timed(c, KC_REDUCE, [&] { return launch_reduce(npart, false, ra, c->stream); });
        if (st) return st;
        for (int q = 0; q < 2 && levels[q] >= 0; ++q) JAC_HIP(hipEventRecord(c->ev[g[q] % kRing], c->stream));
    }
    *buf ^= 1;
    return JAC_OK;
}

// One step through the launch driver for temporal blocking deeper than the
// check interval (D >= 9, D > M): launches of up to D sweeps, each measuring
// the residual of the levels where a check falls (at most two per launch),
// checks every M sweeps as the oracle does.  A check that stops the step at an
// inner level c of a launch leaves its result unstored: the launch's input
// u_k is intact (every later launch returns at once on the stop flag), so a
// redo launch of c sweeps from it produces u_{k+c}.  A launch ends on any
// check predicted to stop (which then runs as a residual pass on the exact
// iterate, as in run_step) and on the last allowed check.
int run_step_deep(jac_ctx* c, const jac_opts* o, int64_t* sweeps_out, float* rho_out) {
    const int64_t L = o->M;
    const int D = o->D;
    // sweeps this step may run: launches end on the last allowed check (below
    // max_sweeps + L), one launch of D beyond a stopping check, a redo
    c->fast_now = division_path(c, 1, (double)o->max_sweeps + (double)L + 2.0 * (double)D);
    c->step_serial += 1;
    c->cur_group = -1;
    c->cur_first = false;
    if (c->prof_every > 0) {
        int s0 = drain_profile(c, c->step_serial - 1);
        if (s0) return s0;
    }
    const bool fuse_rhs = c->fast_now != 0;
    int st = fuse_rhs ? JAC_OK : enqueue_rhs(c, o);
    if (st) return st;
    int buf = c->cur;
    int64_t launch_no = 0;  // profiling group of each launch
    // the first launch: L sweeps (it may form b), no check inside
    c->cur_group = launch_no++;
    c->cur_first = true;
    c->rhs_pending = fuse_rhs;
    st = enqueue_sweeps(c, o, L, false, 0, &buf);
    c->rhs_pending = false;
    if (st) return st;
    int64_t k = L;           // sweeps enqueued; u_k is in u[buf]
    int64_t g_next = 1;      // the first check not yet enqueued (g_next * L >= k)
    const int64_t gmax = (o->max_sweeps + L - 1) / L;  // the last allowed check
    bool final_enqueued = false;
    int64_t predicted = 0;
    CheckHistory hist;
    struct Pending {
        int buf;            // the buffer holding the input of the launch that measured it
        int level;          // its level in that launch (0: the input itself)
        int64_t launch;     // that launch's profiling group
        bool sampled;       // measured on every sample_rows-th row: a lower bound of R
    };
    Pending info[kRing];
    auto stops_here = [&](int64_t g) {
        return g >= gmax || hist.predicts_stop(g, o->tol, c->predict_margin);
    };
    // Checks far from the stop measure a sample of the rows, only where no
    // residual can be NaN or overflow (every iterate and b bounded by Ub, as
    // for the constant-divisor path), so that a sample >= tol decides exactly
    // what the whole residual would.
    double Ub = 0.0;
    const bool may_sample =
        c->sample_rows > 1 && c->fast_now &&
        division_path(c, 1, (double)o->max_sweeps + (double)L + 2.0 * (double)D, &Ub) &&
        (8.0 + 8.0 * (double)c->r) * Ub * 1.001 < (double)FLT_MAX;
    auto sampled = [&](int64_t g) {
        return may_sample && !stops_here(g) && !hist.predicts_stop(g, o->tol, kSampleFar) &&
               !(c->prev_sweeps > 0 && g * L >= c->prev_sweeps - 2 * L);
    };
    auto enqueue_more = [&]() -> int {
        const int64_t gk = g_next;
        if (gk * L == k && stops_here(gk)) {
            // measure only, keep u_{gL} in place
            const int slot = (int)((gk - 1) % kRing);
            c->mail->R[slot] = kEmpty;
            c->cur_group = launch_no++;
            c->cur_first = true;
            int s2 = enqueue_residual(c, o, buf, slot);
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[gk % kRing], c->stream));
            info[gk % kRing] = Pending{buf, 0, c->cur_group, false};
            final_enqueued = true;
            if (gk < gmax) predicted = gk;
            g_next = gk + 1;
            return JAC_OK;
        }
        // a launch from k: at most two checks inside, and it ends on a check
        // that stops here
        int64_t m = std::min<int64_t>(D, gk * L - k + 2 * L);
        for (int64_t g = gk; g * L < k + m; ++g)
            if (g * L > k && stops_here(g)) {
                m = g * L - k;
                break;
            }
        if (m <= 8) m = std::min<int64_t>(m, gk * L == k ? L : gk * L - k);  // the shallow kernels check only their input
        int levels[2] = {-1, -1};
        int64_t gs[2] = {0, 0};
        int sm[2] = {0, 0};
        int n = 0;
        for (int64_t g = gk; g * L < k + m && n < 2; ++g, ++n) {
            levels[n] = (int)(g * L - k);
            gs[n] = g;
            sm[n] = sampled(g) ? c->sample_rows - 1 : 0;
            c->mail->R[(g - 1) % kRing] = kEmpty;
        }
        c->cur_group = launch_no++;
        c->cur_first = true;
        const int in_buf = buf;
        int s2 = enqueue_tb_deep(c, o, (int)m, levels, gs, false, &buf, sm);
        if (s2) return s2;
        for (int q = 0; q < n; ++q)
            info[gs[q] % kRing] = Pending{in_buf, levels[q], c->cur_group, sm[q] != 0};
        k += m;
        g_next = gk + n;
        return JAC_OK;
    };

    for (int64_t g = 1;; ++g) {
        while (!final_enqueued && g_next <= g + 1) {  // keep one check queued beyond check g
            st = enqueue_more();
            if (st) return st;
        }
        const int ev = (int)(g % kRing);
        const int slot = (int)((g - 1) % kRing);
        JAC_HIP(hipEventSynchronize(c->ev[ev]));
        const uint32_t Rb = await_mail(c, &c->mail->R[slot]);
        if (Rb == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
        const float R = mail_float(&c->mail->R[slot]);
        const float rho = R / mail_float(&c->mail->bA_bits);
        const int64_t kk = g * L;
        const bool stop = !(rho >= o->tol);
        if (stop || kk >= o->max_sweeps) {
            const Pending p = info[ev];
            // every launch queued behind the check returned at once (stop flag)
            if (c->prof_every > 0 && stop) mark_noops(c, p.launch);
            // u_{gL}: the intact input, or p.level sweeps past it (a redo)
            int b2 = p.buf;
            if (p.level > 0) {
                const int none[2] = {-1, -1};
                const int64_t g0[2] = {0, 0};
                c->cur_group = p.launch;
                c->cur_first = true;
                st = enqueue_tb_deep(c, o, p.level, none, g0, true, &b2);
                if (st) return st;
            }
            float rho_f = rho;
            if (p.sampled) {
                // a sample below tol decides nothing: the whole residual of
                // u_{gL}, with the stop flag cleared (behind the launches that
                // returned at once) so that its reduction reports
                JAC_HIP(launch_fill(reinterpret_cast<float*>(&c->sc->stop), 1, 0.0f, c->stream));
                c->mail->R[slot] = kEmpty;
                c->cur_group = p.launch;
                c->cur_first = false;
                st = enqueue_residual(c, o, b2, slot);
                if (st) return st;
                JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
                JAC_HIP(hipEventSynchronize(c->ev[ev]));
                if (await_mail(c, &c->mail->R[slot]) == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
                rho_f = mail_float(&c->mail->R[slot]) / mail_float(&c->mail->bA_bits);
                c->verified += 1;
                if (rho_f >= o->tol) {
                    // the step goes on from u_{gL}
                    buf = b2;
                    k = kk;
                    g_next = g + 1;
                    final_enqueued = false;
                    predicted = 0;
                    hist.push(g, rho_f);
                    continue;
                }
            }
            for (int64_t i = 0; i < g; ++i) c->dlog.push_back(D);
            c->cur = b2;
            c->prev_sweeps = kk;
            if (sweeps_out) *sweeps_out = kk;
            if (rho_out) *rho_out = rho_f;
            if (std::isnan(rho_f)) return fail(JAC_ENAN, "rho is NaN");
            if (rho_f >= o->tol) return fail(JAC_ENOCONV, "max_sweeps reached before rho < tol");
            return JAC_OK;
        }
        hist.push(g, rho);
        if (g == predicted) {
            // the predicted final check did not converge: launches go on from u_{gL}
            final_enqueued = false;
            predicted = 0;
        }
        if (c->prof_every > 0 && c->recs.size() > 8192) {
            st = drain_profile(c, c->step_serial);
            if (st) return st;
        }
    }
}

// One step through the launch or the graph driver.  Check g (g >= 1) examines
// u_{gL}; its R lands in mailbox slot (g - 1) % kRing.
int run_step(jac_ctx* c, const jac_opts* o, int64_t* sweeps_out, float* rho_out) {
    if (o->checks == JAC_CHECKS_BLOCKING || o->controller != JAC_STATIC)
        return run_step_blocking(c, o, sweeps_out, rho_out);
    if (o->kernel == JAC_TBLOCK && o->driver == JAC_LAUNCH && o->D >= 9 && o->D > o->M)
        return run_step_deep(c, o, sweeps_out, rho_out);
    const int64_t L = check_interval(o);
    const bool graph = o->driver == JAC_GRAPH;
    // sweeps this step may run: up to max_sweeps, plus the interval queued beyond a check
    c->fast_now = division_path(c, 1, (double)o->max_sweeps + 2.0 * (double)L);
    c->step_serial += 1;
    c->cur_group = -1;
    c->cur_first = false;
    if (c->prof_every > 0) {
        int s0 = drain_profile(c, c->step_serial - 1);  // earlier steps have finished
        if (s0) return s0;
    }
    // temporal blocking through the launch driver forms b in the step's first
    // launch; the other paths run the separate right-hand-side pass
    const bool fuse_rhs = !graph && o->kernel == JAC_TBLOCK && c->fast_now;
    int st = fuse_rhs ? JAC_OK : enqueue_rhs(c, o);
    if (st) return st;
    int buf = c->cur;
    c->cur_group = 0;
    c->cur_first = true;
    if (graph) {  // group 0: sweeps 1..L
        hipGraphExec_t gx;
        int flips;
        st = graph_for(c, o, false, buf, &gx, &flips);
        if (st) return st;
        JAC_HIP(hipGraphLaunch(gx, c->stream));
        buf ^= flips;
    } else {
        c->rhs_pending = fuse_rhs;
        st = enqueue_sweeps(c, o, L, false, 0, &buf);
        c->rhs_pending = false;
        if (st) return st;
    }

    int64_t g_enq = 1;  // next group to enqueue
    bool final_enqueued = false;
    int64_t predicted = 0;  // the check queued alone on a prediction (0: none)
    CheckHistory hist;
    // Temporal-blocking launches measure checks far from the stop on a sample
    // of the rows, as run_step_deep does (same bound, same policy)
    double Ub = 0.0;
    const bool may_sample =
        !graph && c->sample_rows > 1 &&
        (o->kernel == JAC_TBLOCK ||
         (o->kernel == JAC_ASYNC && c->sample_rows == 8 &&
          async_samples_rows(c->N, o->tile_x, o->tile_y, o->overlap, o->D))) &&
        c->fast_now &&
        division_path(c, 1, (double)o->max_sweeps + 2.0 * (double)L, &Ub) &&
        (8.0 + 8.0 * (double)c->r) * Ub * 1.001 < (double)FLT_MAX;
    bool samp[kRing] = {};
    auto sampled = [&](int64_t g) {
        return may_sample && !hist.predicts_stop(g, o->tol, kSampleFar) &&
               !(c->prev_sweeps > 0 && g * L >= c->prev_sweeps - 2 * L);
    };
    // the interval after check g, from u_{gL}, without a check (group 0's form)
    auto enqueue_plain_interval = [&](int64_t g) -> int {
        c->cur_group = g;
        c->cur_first = false;
        if (graph) {
            hipGraphExec_t gx;
            int flips;
            int s2 = graph_for(c, o, false, buf, &gx, &flips);
            if (s2) return s2;
            JAC_HIP(hipGraphLaunch(gx, c->stream));
            buf ^= flips;
            return JAC_OK;
        }
        return enqueue_sweeps(c, o, L, false, 0, &buf);
    };
    auto enqueue_group = [&]() -> int {
        const int ev = (int)(g_enq % kRing);
        const int slot = (int)((g_enq - 1) % kRing);
        c->start_buf[ev] = buf;
        c->mail->R[slot] = kEmpty;
        c->cur_group = g_enq;
        c->cur_first = true;
        samp[ev] = false;
        int s2;
        if (g_enq * L >= o->max_sweeps) {
            // the last allowed check: measure only, keep u_{gL} in place
            s2 = enqueue_residual(c, o, buf, slot);
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
            final_enqueued = true;
        } else if (hist.predicts_stop(g_enq, o->tol, c->predict_margin)) {
            // predicted to end the step: measure only, keep u_{gL} in place
            s2 = enqueue_residual(c, o, buf, slot);
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
            final_enqueued = true;
            predicted = g_enq;
        } else if (graph) {
            hipGraphExec_t gx;
            int flips;
            s2 = graph_for(c, o, true, buf, &gx, &flips);
            if (s2) return s2;
            JAC_HIP(hipGraphLaunch(gx, c->stream));
            JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
            buf ^= flips;
        } else {
            // one launch that checks u_{gL} and starts the next interval, then the rest
            const int64_t first = std::min<int64_t>(L, sweeps_per_launch(o));
            samp[ev] = sampled(g_enq);
            c->cur_smask = samp[ev] ? c->sample_rows - 1 : 0;
            s2 = enqueue_sweeps(c, o, first, true, slot, &buf);
            c->cur_smask = 0;
            if (s2) return s2;
            JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
            s2 = enqueue_sweeps(c, o, L - first, false, slot, &buf);
            if (s2) return s2;
        }
        ++g_enq;
        return JAC_OK;
    };

    st = enqueue_group();
    if (st) return st;
    for (int64_t g = 1;; ++g) {
        while (!final_enqueued && g_enq <= g + 1) {  // keep one interval queued beyond check g
            st = enqueue_group();
            if (st) return st;
        }
        const int ev = (int)(g % kRing);
        const int slot = (int)((g - 1) % kRing);
        JAC_HIP(hipEventSynchronize(c->ev[ev]));
        const uint32_t Rb = await_mail(c, &c->mail->R[slot]);
        if (Rb == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
        const float R = mail_float(&c->mail->R[slot]);
        const float rho = R / mail_float(&c->mail->bA_bits);
        const int64_t k = g * L;
        const bool stop = !(rho >= o->tol);
        if (stop || k >= o->max_sweeps) {
            if (c->prof_every > 0 && stop) mark_noops(c, g);
            float rho_f = rho;
            if (samp[ev] && stop) {
                // a sample below tol decides nothing: the whole residual of
                // u_{gL} (intact: every launch behind the check returned at
                // once), with the stop flag cleared so that its reduction reports
                JAC_HIP(launch_fill(reinterpret_cast<float*>(&c->sc->stop), 1, 0.0f, c->stream));
                c->mail->R[slot] = kEmpty;
                c->cur_group = g;
                c->cur_first = false;
                st = enqueue_residual(c, o, c->start_buf[ev], slot);
                if (st) return st;
                JAC_HIP(hipEventRecord(c->ev[ev], c->stream));
                JAC_HIP(hipEventSynchronize(c->ev[ev]));
                if (await_mail(c, &c->mail->R[slot]) == kEmpty) return fail(JAC_EDEVICE, "a residual check did not report");
                rho_f = mail_float(&c->mail->R[slot]) / mail_float(&c->mail->bA_bits);
                c->verified += 1;
                if (rho_f >= o->tol) {
                    // the step goes on: the interval after check g, from u_{gL}
                    buf = c->start_buf[ev];
                    g_enq = g + 1;
                    final_enqueued = false;
                    predicted = 0;
                    hist.push(g, rho_f);
                    st = enqueue_plain_interval(g);
                    if (st) return st;
                    continue;
                }
            }
            for (int64_t i = 0; i < g; ++i) c->dlog.push_back(sweeps_per_launch(o));
            c->cur = c->start_buf[ev];
            c->prev_sweeps = k;
            if (sweeps_out) *sweeps_out = k;
            if (rho_out) *rho_out = rho_f;
            if (std::isnan(rho_f)) return fail(JAC_ENAN, "rho is NaN");
            if (rho_f >= o->tol) return fail(JAC_ENOCONV, "max_sweeps reached before rho < tol");
            return JAC_OK;
        }
        hist.push(g, rho);
        if (g == predicted) {
            // the predicted final check did not converge: the skipped interval next
            st = enqueue_plain_interval(g);
            if (st) return st;
            final_enqueued = false;
            predicted = 0;
        }
        if (c->prof_every > 0 && c->recs.size() > 8192) {
            st = drain_profile(c, c->step_serial);  // keep this step's records (their class may change)
            if (st) return st;
        }
    }
}

// The whole solve in one cooperative kernel: the device runs every step,
// check and decision; the host reads the per-step records at the end.
struct PersistRec {
    int64_t sweeps;
    uint32_t R_bits, bA_bits;
    int32_t status, cur;
};

int run_persistent(jac_ctx* c, const jac_opts* o, int nsteps, int64_t* sweeps, float* rho) {
    if (nsteps == 0) return JAC_OK;
    if (persist_out_bytes() != sizeof(PersistRec)) return fail(JAC_EDEVICE, "persistent record layout mismatch");
    if (nsteps > c->pout_cap) {
        if (c->pout) JAC_HIP(hipHostFree(c->pout));
        c->pout = nullptr;
        c->pout_cap = 0;
        JAC_HIP(hipHostMalloc(&c->pout, sizeof(PersistRec) * (size_t)nsteps, hipHostMallocDefault));
        c->pout_cap = nsteps;
    }
    PersistRec* rec = reinterpret_cast<PersistRec*>(c->pout);
    for (int n = 0; n < nsteps; ++n) rec[n] = PersistRec{0, 0, 0, 1, c->cur};
    const bool async_mode = o->kernel == JAC_ASYNC;
    const int L = (int)check_interval(o);
    // temporal blocking runs chunks of at most one check interval
    const int D = o->kernel == JAC_SYNC ? 1 : (o->kernel == JAC_TBLOCK ? std::min(o->D, L) : o->D);
    c->fast_now = division_path(c, nsteps, (double)o->max_sweeps + 2.0 * (double)L);
    StepArgs a = base_args(c, o->tol);
    int grid = 0;
    c->cur_group = -1;
    int st = timed(c, KC_PERSIST, [&] {
        return launch_persist(a, c->u[0], c->u[1], c->b, c->s, scratch_partials(c->sc), c->xchg,
                              exchange_words_cap(c->g.N), c->pout, nsteps, c->cur, async_mode, D, L, o->tile_x,
                              o->tile_y, o->band_rows, o->max_sweeps, c->cus, &grid, c->stream);
    });
    if (st) return st;
    if (4 * (int64_t)grid > c->npart_cap) return fail(JAC_EDEVICE, "persistent grid exceeds partial slots");
    JAC_HIP(hipStreamSynchronize(c->stream));
    uint32_t bar_error = 0;
    JAC_HIP(hipMemcpy(&bar_error, &c->sc->bar_error, 4, hipMemcpyDeviceToHost));
    if (bar_error) return fail(JAC_EDEVICE, "persistent kernel: a grid barrier wait timed out");
    int status = JAC_OK;
    for (int n = 0; n < nsteps; ++n) {
        const volatile PersistRec* r = &rec[n];
        if (r->status == 1) break;
        float R, bA;
        const uint32_t Rb = r->R_bits, bAb = r->bA_bits;
        std::memcpy(&R, &Rb, 4);
        std::memcpy(&bA, &bAb, 4);
        if (sweeps) sweeps[n] = r->sweeps;
        if (rho) rho[n] = R / bA;
        c->cur = r->cur;
        grow_ubound(c, (double)r->sweeps);
        if (r->status != 0) {
            status = r->status;
            break;
        }
    }
    if (status == JAC_ENAN) return fail(JAC_ENAN, "rho is NaN");
    if (status == JAC_ENOCONV) return fail(JAC_ENOCONV, "max_sweeps reached before rho < tol");
    return JAC_OK;
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
    o->band_rows = 0;
    o->max_sweeps = 1000000;
    o->checks = JAC_CHECKS_OVERLAPPED;
    o->controller = JAC_STATIC;
    o->overlap = 0;
    o->reserved = 0;
}

size_t jac_workspace_bytes(int N) {
    if (N < 1 || N > kMaxN) return 0;
    Geom g = make_geom(N);
    const size_t bytes =
        (size_t)exchange_offset_floats(g, partial_cap(N)) * sizeof(float) + (size_t)exchange_words_cap(N) * 8;
    return (bytes + 255) / 256 * 256;
}

const char* jac_last_error(void) { return g_err.c_str(); }

// Between calls the iterate plane other than u_cur holds nothing a later call
// reads: the next sweep writes all of its unknowns before any is read.  Host
// transfers stage the N x N field there as one contiguous block -- one 1-D
// copy (a pitched copy from pageable host memory ran several times slower)
// and a pitch-changing kernel -- and then restore the plane to what every
// sweep expects of its ghost ring and padding: zeros, the top ghost row 100.
static hipError_t restore_plane(jac_ctx* c, int k) {
    hipError_t e = launch_fill(c->u[k], c->g.plane, 0.0f, c->stream);
    if (e == hipSuccess) e = launch_ghosts(c->u[k], c->g, c->stream);
    return e;
}

// host_in (N x N, row-major) into the unknowns of plane dst, through plane
// u[stage]; stream-ordered, host_in must stay valid until the stream is synced
static hipError_t upload_block(jac_ctx* c, float* dst, const float* host_in, int stage) {
    hipError_t e = hipMemcpyAsync(c->u[stage], host_in, (size_t)c->N * c->N * 4, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = launch_copy_rect(dst + c->g.origin, c->g.P, c->u[stage], c->N, c->N, c->stream);
    return e;
}

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
        c->y = 1.0f / c->d;  // correctly rounded on the host (SSE division)
    }
    c->fastdiv = 0;
    c->fast_now = 0;
    c->graph_fast = -1;
    c->ubound = 100.0;  // u^0 = 0 and the top ghost row
    c->smax = 0.0;
    c->src_plain = true;
    if (source_host) {
        // max |s| as the largest magnitude bit pattern (Inf and NaN sit above
        // every finite value), and whether any element is -0: one pass the
        // compiler vectorises
        const uint32_t* w = reinterpret_cast<const uint32_t*>(source_host);
        uint32_t mb = 0, negz = 0;
        for (int64_t i = 0; i < (int64_t)N * N; ++i) {
            const uint32_t a = w[i] & 0x7fffffffu;
            mb = a > mb ? a : mb;
            negz |= (uint32_t)(w[i] == 0x80000000u);
        }
        float mf;
        std::memcpy(&mf, &mb, 4);
        c->src_plain = mb < 0x7f800000u && !negz;
        c->smax = mb < 0x7f800000u ? (double)mf : (double)INFINITY;
    }
    c->cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    c->sync_rows = sync_rows_for(N, c->cus);
    c->pout = nullptr;
    c->pout_cap = 0;
    c->cap_stream = nullptr;
    c->graphs_valid = false;
    for (int i = 0; i < 2; ++i) { c->g_first[i] = nullptr; c->g_group[i] = nullptr; }
    c->g_flips_first = c->g_flips_group = 0;
    for (int i = 0; i <= kMaxTBlockD; ++i) c->tb_rows[i] = 0;
    c->g = make_geom(N);
    c->stream = (hipStream_t)stream;
    float* base = (float*)workspace;
    c->u[0] = base;
    c->u[1] = base + c->g.plane;
    c->b = base + 2 * c->g.plane;
    c->s = base + 3 * c->g.plane;
    c->sc = (Scratch*)(base + 4 * c->g.plane);
    c->npart_cap = partial_cap(N);
    c->xchg = reinterpret_cast<uint64_t*>(base + exchange_offset_floats(c->g, c->npart_cap));
    c->static_sc = nullptr;
    c->static_err = hipErrorInvalidDevice;
    if (dev >= 0 && dev < kMaxDevices) {
        // once per device, with that device current: the device address of the
        // static scratch array (each GPU holds its own copy)
        // (a failed lookup is reported by jac_sweep_static, not here: the
        // context itself does not need the array)
        std::lock_guard<std::mutex> lock(g_static_mu);
        if (!g_static_sc[dev] && g_static_err[dev] == hipSuccess) {
            void* ptr = nullptr;
            const hipError_t se = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (se == hipSuccess && ptr)
                g_static_sc[dev] = (Scratch*)ptr;
            else
                g_static_err[dev] = se != hipSuccess ? se : hipErrorInvalidSymbol;
        }
        c->static_sc = g_static_sc[dev];
        c->static_err = g_static_err[dev];
    }
    c->cur = 0;
    c->rhs_pending = false;
    {
        // JACOBI_PREDICT_MARGIN=m at create time: m = 0 turns the final-check
        // prediction off; results never depend on it
        const char* pm = std::getenv("JACOBI_PREDICT_MARGIN");
        const float m = pm ? std::strtof(pm, nullptr) : kPredictMargin;
        c->predict_margin = (std::isfinite(m) && m > 0.0f) ? m : 0.0f;
        // JACOBI_SAMPLED_CHECKS=n at create time: the row stride of the
        // residual a deep temporal-blocking launch takes at a check that is
        // not expected to stop (a power of two; 0 or 1: every row)
        const char* sr = std::getenv("JACOBI_SAMPLED_CHECKS");
        long n = sr ? std::strtol(sr, nullptr, 10) : (long)kSampleRows;
        c->sample_rows = (n >= 2 && n <= (1L << 20) && (n & (n - 1)) == 0) ? (int)n : 0;
        c->prev_sweeps = 0;
        c->verified = 0;
        c->cur_smask = 0;
    }
    c->prof_every = 0;
    c->step_serial = 0;
    c->cur_group = -1;
    c->cur_first = false;
    for (int i = 0; i < kClasses; ++i) { c->ms[i] = 0.0; c->cnt[i] = 0; c->seen[i] = 0; c->timed_n[i] = 0; }
    for (int i = 0; i < kRing; ++i) c->ev[i] = nullptr;
    c->mail = nullptr;

    auto cleanup_fail = [&](int code) {
        jac_destroy(c);
        return code;
    };
    if (hipHostMalloc((void**)&c->mail, sizeof(Mailbox), hipHostMallocCoherent) != hipSuccess)
        return cleanup_fail(fail(JAC_ENOMEM, "hipHostMalloc of the result mailbox failed"));
    std::memset(c->mail, 0xFF, sizeof(Mailbox));
    // Check events only tell the host that a check's reduction has run; its
    // result reaches the host through the coherent mailbox, so they skip the
    // system-scope fence (a cache writeback that would stall the next kernel
    // by ~5 us after every check).
    for (int i = 0; i < kRing; ++i)
        if (hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
            return cleanup_fail(fail(JAC_EDEVICE, "hipEventCreateWithFlags failed"));

    hipError_t e = launch_fill(base,
                               c->g.plane * 4 + (int64_t)(sizeof(Scratch) / 4) +
                                   (int64_t)kMaxPersistBlocks * kFlagStride + c->npart_cap,
                               0.0f, c->stream);
    // the source goes through u_1 (idle until the first sweep) as one block
    if (e == hipSuccess && source_host) e = upload_block(c, c->s, source_host, 1);
    if (e == hipSuccess) e = launch_fill(c->u[1], c->g.plane, 0.0f, c->stream);
    if (e == hipSuccess) e = launch_ghosts(c->u[0], c->g, c->stream);
    if (e == hipSuccess) e = launch_ghosts(c->u[1], c->g, c->stream);
    // The sweep divides by the constant d.  Use the reciprocal-and-correct
    // quotient only if it equals the IEEE quotient on every float input.
    const char* ieee_env = std::getenv("JACOBI_IEEE_DIVISION");
    const bool want_fast = !(ieee_env && ieee_env[0] == '1');
    if (e == hipSuccess && want_fast) e = launch_verify_div(c->d, c->y, c->sc, c->stream);
    uint32_t bad = 1;
    if (e == hipSuccess && want_fast)
        e = hipMemcpyAsync(&bad, &c->sc->div_bad, 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return cleanup_fail(fail(JAC_EDEVICE, std::string("set-up: ") + hipGetErrorString(e)));
    c->fastdiv = (want_fast && bad == 0) ? 1 : 0;
    *out = c;
    return JAC_OK;
}

int jac_destroy(jac_t c) {
    if (!c) return JAC_OK;
    (void)hipStreamSynchronize(c->stream);
    for (int i = 0; i < kRing; ++i)
        if (c->ev[i]) (void)hipEventDestroy(c->ev[i]);
    for (Rec& p : c->recs) {
        if (p.e0) (void)hipEventDestroy(p.e0);
        if (p.e1) (void)hipEventDestroy(p.e1);
    }
    for (hipEvent_t e : c->free_ev) (void)hipEventDestroy(e);
    if (c->mail) (void)hipHostFree(c->mail);
    if (c->pout) (void)hipHostFree(c->pout);
    for (int i = 0; i < 2; ++i) {
        if (c->g_first[i]) (void)hipGraphExecDestroy(c->g_first[i]);
        if (c->g_group[i]) (void)hipGraphExecDestroy(c->g_group[i]);
    }
    if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
    delete c;
    return JAC_OK;
}

int jac_step(jac_t c, const jac_opts* o, int64_t* sweeps, float* rho) { return jac_solve(c, 1, o, sweeps, rho); }

int jac_solve(jac_t c, int nsteps, const jac_opts* o, int64_t* sweeps, float* rho) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (nsteps < 0) return fail(JAC_EINVAL, "nsteps must be >= 0");
    int st = check_opts(c, o);
    if (st) return st;
    // a block-async check takes one partial-maximum slot per block, and the
    // launch forms run one block per tile: tiles far smaller than 64 points
    // on a large grid would fail at the first check, after work had run
    if (o->kernel == JAC_ASYNC && o->driver != JAC_PERSISTENT &&
        async_blocks(c->N, o->tile_x, o->tile_y, o->overlap) > c->npart_cap)
        return fail(JAC_EINVAL, "tile too small for this N: more blocks than partial-maximum slots");
    for (int n = 0; n < nsteps; ++n) {
        if (sweeps) sweeps[n] = 0;
        if (rho) rho[n] = NAN;
    }
    c->dlog.clear();
    if (o->driver == JAC_PERSISTENT) {
        st = run_persistent(c, o, nsteps, sweeps, rho);
    } else {
        for (int n = 0; n < nsteps; ++n) {
            int64_t k = 0;
            st = run_step(c, o, &k, rho ? &rho[n] : nullptr);
            if (sweeps) sweeps[n] = k;
            grow_ubound(c, (double)(k > 0 ? k : o->max_sweeps));
            if (st) break;
        }
    }
    if (st == JAC_ENAN || st == JAC_EDEVICE) c->ubound = INFINITY;  // the field may hold anything
    if (c->prof_every > 0) {
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
    c->step_serial += 1;
    c->cur_group = -1;
    c->cur_first = false;
    c->fast_now = division_path(c, 1, (double)nsweeps);
    st = enqueue_rhs(c, o);
    if (st) return st;
    int buf = c->cur;
    st = enqueue_sweeps(c, o, nsweeps, false, 0, &buf);
    if (st) {
        c->ubound = INFINITY;
        return st;
    }
    c->cur = buf;
    grow_ubound(c, (double)nsweeps);
    if (rho) {
        c->mail->R[0] = kEmpty;
        st = enqueue_residual(c, o, c->cur, 0);
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
    if (c->prof_every > 0) return drain_profile(c);
    return JAC_OK;
}

int jac_sweep_static(jac_t c, const jac_opts* o, int64_t nsweeps, float* rho) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (!c->static_sc)
        return fail(JAC_EDEVICE, std::string("no static scratch on this context's device: hipGetSymbolAddress: ") +
                                     hipGetErrorString(c->static_err));
    if (c->N > kStaticMaxN) return fail(JAC_EINVAL, "jac_sweep_static supports N up to 16384");
    int st = check_opts(c, o);
    if (st) return st;
    // every reducing launch of jac_sweep must fit the static partial slots
    int64_t need = std::max(rhs_blocks(c->N), sync_blocks(c->N, c->sync_rows));
    if (need > kStaticPartials)
        return fail(JAC_EINVAL, "jac_sweep_static: the launch needs more than 32768 partial slots");
    // jac_sweep with the static scratch and the launch timer off (its records
    // are the only host allocations jac_sweep makes); everything else -- the
    // kernels, the field, the caller's workspace planes -- is the same
    Scratch* const saved_sc = c->sc;
    const int64_t saved_cap = c->npart_cap;
    const int saved_prof = c->prof_every;
    c->sc = c->static_sc;
    c->npart_cap = kStaticPartials;
    c->prof_every = 0;
    st = jac_sweep(c, o, nsweeps, rho);
    c->sc = saved_sc;
    c->npart_cap = saved_cap;
    c->prof_every = saved_prof;
    return st;
}

int jac_get_field(jac_t c, float* host_out) {
    if (!c || !host_out) return fail(JAC_EINVAL, "NULL argument");
    // u_cur's unknowns packed into the idle plane, one 1-D copy out, the
    // idle plane restored
    // idle plane restored even when the copy out fails (a bad host pointer)
    const int idle = 1 - c->cur;
    hipError_t e = launch_copy_rect(c->u[idle], c->N, c->u[c->cur] + c->g.origin, c->g.P, c->N, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(host_out, c->u[idle], (size_t)c->N * c->N * 4, hipMemcpyDeviceToHost, c->stream);
    const hipError_t er = restore_plane(c, idle);
    if (e == hipSuccess) e = er;
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("jac_get_field: ") + hipGetErrorString(e));
    return JAC_OK;
}

int jac_set_field(jac_t c, const float* host_in) {
    if (!c || !host_in) return fail(JAC_EINVAL, "NULL argument");
    c->ubound = INFINITY;
    // max(100, max |u|) (100: the top ghost row), or Inf if any value is not
    // finite: |x| compared as the bits of a non-negative float, where NaN and
    // Inf sit above every finite value
    const uint32_t* w = reinterpret_cast<const uint32_t*>(host_in);
    uint32_t mb = 0;
    for (int64_t i = 0; i < (int64_t)c->N * c->N; ++i) {
        const uint32_t a = w[i] & 0x7fffffffu;
        mb = a > mb ? a : mb;
    }
    float mf;
    std::memcpy(&mf, &mb, 4);
    const double m = mb >= 0x7f800000u ? (double)INFINITY : std::max(100.0, (double)mf);
    hipError_t e = upload_block(c, c->u[c->cur], host_in, 1 - c->cur);
    const hipError_t er = restore_plane(c, 1 - c->cur);  // also after a failed copy in
    if (e == hipSuccess) e = er;
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(JAC_EDEVICE, std::string("jac_set_field: ") + hipGetErrorString(e));
    c->ubound = m;
    return JAC_OK;
}

int jac_reset(jac_t c) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    JAC_HIP(launch_fill(c->u[0], c->g.plane * 2, 0.0f, c->stream));
    JAC_HIP(launch_ghosts(c->u[0], c->g, c->stream));
    JAC_HIP(launch_ghosts(c->u[1], c->g, c->stream));
    c->cur = 0;
    JAC_HIP(hipStreamSynchronize(c->stream));
    c->ubound = 100.0;
    c->prev_sweeps = 0;
    return JAC_OK;
}

int jac_stream_probe(float* c, const float* a, const float* b, size_t n, int kind, int nontemporal,
                     int blocks, void* stream) {
    if (!c || !a || (kind == 1 && !b)) return fail(JAC_EINVAL, "NULL array");
    if (kind != 0 && kind != 1) return fail(JAC_EINVAL, "kind must be 0 (copy) or 1 (add)");
    if (n % 4 != 0 || ((uintptr_t)a | (uintptr_t)c | (uintptr_t)(b ? b : a)) % 16 != 0)
        return fail(JAC_EINVAL, "n must be a multiple of 4 and the arrays 16-byte aligned");
    if (blocks < 1 || blocks > (1 << 20)) return fail(JAC_EINVAL, "blocks must be in 1..2^20");
    JAC_HIP(launch_probe(c, a, b, (int64_t)n, kind, nontemporal != 0, blocks, (hipStream_t)stream));
    return JAC_OK;
}

int jac_fast_division(jac_t c) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    return c->fastdiv;
}

int jac_depth_log(jac_t c, int32_t* depths, int64_t cap, int64_t* count) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (cap < 0 || (cap > 0 && !depths)) return fail(JAC_EINVAL, "depths is NULL or cap < 0");
    const int64_t n = (int64_t)c->dlog.size();
    for (int64_t i = 0; i < n && i < cap; ++i) depths[i] = c->dlog[(size_t)i];
    if (count) *count = n;
    return JAC_OK;
}

int jac_last_division(jac_t c) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    return c->fast_now;
}

int jac_profile(jac_t c, int every) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (every < 0) return fail(JAC_EINVAL, "every must be >= 0");
    int st = drain_profile(c);
    if (st) return st;
    c->prof_every = every;
    for (int i = 0; i < kClasses; ++i) { c->ms[i] = 0.0; c->cnt[i] = 0; c->seen[i] = 0; c->timed_n[i] = 0; }
    return JAC_OK;
}

int jac_profile_read(jac_t c, int kclass, double* ms_timed, int64_t* launches, int64_t* timed_launches) {
    if (!c) return fail(JAC_EINVAL, "context is NULL");
    if (kclass < 0 || kclass >= kClasses) return fail(JAC_EINVAL, "unknown kernel class");
    int st = drain_profile(c);
    if (st) return st;
    if (ms_timed) *ms_timed = c->ms[kclass];
    if (launches) *launches = c->cnt[kclass];
    if (timed_launches) *timed_launches = c->timed_n[kclass];
    return JAC_OK;
}

}  // extern "C"
