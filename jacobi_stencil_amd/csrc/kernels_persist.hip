// kernels_persist.hip -- the whole solve in one cooperative kernel.
//
// For grids that fit the on-chip caches the time per sweep is set by launch
// latency and by the host deciding convergence, not by memory (page
// "stencil-jacobian.vercel.app", section 04: the synchronisation that costs
// time is the host round trip).  A persistent kernel keeps the time loop, the
// residual and the convergence decision on the device (the CPU-free model of
// the paperlayer summary of arXiv 2610.15878, sections 3-4: persistent
// kernels, device-side barriers, no host in the loop).
//
// Every block runs the same program:
//   per step:   b = u^n + s and a partial max of |b_A|;  grid barrier;  every
//               block reduces the partials to ||b_A|| (the same value in all)
//   per chunk:  for each of its tiles, stage the tile plus an H-cell halo of
//               u_k in LDS, do Dc sweeps there, store the tile's core to the
//               other buffer;  grid barrier.  A chunk that starts at a check
//               point (k = gL, g >= 1) first measures the residual of u_k on the
//               tile cores; after the barrier every block reduces the partials
//               and takes the same decision.  A stop keeps u_k (the chunk's
//               output is discarded).
// Two tile programs:
//   exact (SYNC, TBLOCK): H = Dc, sweep s updates the cells at least s cells
//     inside the staged edge (ghost-zone temporal blocking; page section 02);
//     after Dc sweeps the core equals Dc synchronous sweeps bit for bit.
//   async (ASYNC): H = 1, every sweep updates the whole tile, the halo stays
//     frozen -- exactly one block-asynchronous launch.
// Ghost cells and padding never change, so both LDS buffers hold them as
// staged.  Every block makes the same decisions from the same reduced values,
// so all reach the same barriers and leave together; max_sweeps bounds every
// loop.
#include "jacobi_internal.h"

namespace jac {

constexpr int kPersistThreads = 1024;
constexpr int kPersistMaxCells = 8192;  // staged region (tile + 2H cells per side) at most: 2 x 32 KB of LDS
constexpr int kPersistCellsPerThread = (kPersistMaxCells + kPersistThreads - 1) / kPersistThreads;

struct PersistOut {
    int64_t sweeps;
    uint32_t R_bits;
    uint32_t bA_bits;
    int32_t status;  // JAC_OK, JAC_ENOCONV, JAC_ENAN; 1: not run
    int32_t cur;     // buffer holding the step's result
};

struct PersistArgs {
    Geom g;
    float r, d, y, tol;
    float* u0;
    float* u1;
    float* b;
    const float* s;
    uint32_t* partial;   // 2 x gridDim.x slots (double-buffered)
    PersistOut* out;     // nsteps records, pinned host memory
    int nsteps, cur0;
    int async_mode;      // 0: exact tiles (ghost zone), 1: block-asynchronous tiles
    int D, L;            // sweeps per chunk, check interval
    int tx, ty;          // tile core
    int lds_cells;       // staged region of the deepest chunk; the second LDS buffer starts there
    int64_t max_sweeps;
    Scratch* sc;         // barrier words (cleared by the host before the launch)
};

// Spin budget of one barrier wait: ~0.1 us per poll, about a second in all.
constexpr uint32_t kBarrierSpins = 10000000u;

// Grid-wide barrier over all blocks (all co-resident: cooperative launch), with
// no contended atomics: every block stores its new generation to its own flag
// line; block 0's threads wait for all flags, then block 0 stores the
// generation to the release word, which the other blocks wait for.  A wait
// that outlasts the spin budget sets the error word; every waiter polls it, so
// all blocks leave.  Returns false when the kernel must stop.  `gen` counts
// this block's barriers (the host zeroed the flags and the release word).
// Memory order: one device-scope release per store (each one writes back the
// XCD's L2, so there is no extra fence beside it), relaxed polls, and one
// acquire after a wait -- an acquiring poll would invalidate the cache on
// every spin (N = 256, ten steps: 18.1 -> 15.9 ms for the synchronous sweep,
// 4.47 -> 4.01 ms for temporal blocking at D = 8).
__device__ bool grid_barrier(Scratch* sc, uint32_t& gen) {
    __shared__ uint32_t ok;
    const uint32_t next = gen + 1;
    uint32_t* flags = scratch_flags(sc);
    __syncthreads();  // the block's writes before thread 0's release below
    if (threadIdx.x == 0) {
        __hip_atomic_store(&flags[(size_t)blockIdx.x * kFlagStride], next, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
        ok = 1;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        // each thread watches some of the flags (relaxed polls, one acquire after)
        uint32_t good = 1;
        for (int i = threadIdx.x; i < (int)gridDim.x && good; i += blockDim.x) {
            uint32_t spins = 0;
            while (__hip_atomic_load(&flags[(size_t)i * kFlagStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   next) {
                if (__hip_atomic_load(&sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                    ++spins > kBarrierSpins) {
                    __hip_atomic_store(&sc->bar_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    good = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (!good) ok = 0;  // any thread that gave up
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(&sc->bar_release, next, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else if (threadIdx.x == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(&sc->bar_release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < next) {
            if (__hip_atomic_load(&sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                ++spins > kBarrierSpins) {
                __hip_atomic_store(&sc->bar_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other blocks' writes after the barrier
    }
    if (threadIdx.x == 0 && __hip_atomic_load(&sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) ok = 0;
    __syncthreads();
    gen = next;
    return ok != 0;
}

__device__ __forceinline__ void publish_partial(uint32_t* slot, uint32_t v) {
    __hip_atomic_store(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// max over the G partials of buffer `which`, the same in every block
__device__ uint32_t reduce_partials(const uint32_t* partial, int which) {
    __shared__ uint32_t wmax[kPersistThreads / 64];
    const int G = gridDim.x;
    uint32_t m = 0;
    for (int i = threadIdx.x; i < G; i += kPersistThreads) {
        const uint32_t v = __hip_atomic_load(&partial[(int64_t)which * G + i], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        m = m > v ? m : v;
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t r = wmax[0];
    for (int w = 1; w < kPersistThreads / 64; ++w) r = r > wmax[w] ? r : wmax[w];
    __syncthreads();
    return r;
}

// Block max of m, stored to this block's slot of buffer `which`.
__device__ void block_partial(uint32_t m, uint32_t* partial, int which) {
    __shared__ uint32_t wmax[kPersistThreads / 64];
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = wmax[0];
        for (int w = 1; w < kPersistThreads / 64; ++w) r = r > wmax[w] ? r : wmax[w];
        publish_partial(&partial[(int64_t)which * gridDim.x + blockIdx.x], r);
    }
    __syncthreads();
}

// One tile: stage, optionally measure the residual of the staged u_k, Dc
// sweeps, store the core.  Returns the tile's max |res| bits (0 without check).
template <bool FAST>
__device__ uint32_t persist_tile(const PersistArgs& a, const float* __restrict__ uin, float* __restrict__ uout,
                                 int tile, int Dc, bool check, float* lds) {
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int ntx = (N + a.tx - 1) / a.tx;
    const int x0 = (tile % ntx) * a.tx, y0 = (tile / ntx) * a.ty;
    const int w = (x0 + a.tx <= N) ? a.tx : N - x0;
    const int h = (y0 + a.ty <= N) ? a.ty : N - y0;
    const int H = a.async_mode ? 1 : Dc;
    const int lp = w + 2 * H, lh = h + 2 * H;
    const int ncell = lp * lh;
    float* A = lds;
    float* B = lds + a.lds_cells;
    const float r = a.r, d = a.d, y = a.y;
    // cells of this thread: k = threadIdx.x + q * blockDim; (ra, ca) by a
    // multiply-high division by lp (exact: ncell * lp < 2^32 / lp here)
    const uint32_t magic = (uint32_t)(0xFFFFFFFFull / (uint32_t)lp) + 1u;
    int ra[kPersistCellsPerThread], ca[kPersistCellsPerThread];
    float bv[kPersistCellsPerThread];
    bool unk[kPersistCellsPerThread];
    const float* su = uin + g.origin + (int64_t)(y0 - H) * P + (x0 - H);
    const float* sb = a.b + g.origin + (int64_t)(y0 - H) * P + (x0 - H);
#pragma unroll
    for (int q = 0; q < kPersistCellsPerThread; ++q) {
        const int k = threadIdx.x + q * kPersistThreads;
        ra[q] = -1;
        ca[q] = -1;
        bv[q] = 0.0f;
        unk[q] = false;
        if (k < ncell) {
            const int rr = (int)__umulhi((uint32_t)k, magic);
            const int cc = k - rr * lp;
            ra[q] = rr;
            ca[q] = cc;
            const float v = su[(int64_t)rr * P + cc];
            A[k] = v;
            B[k] = v;
            const int gi = y0 - H + rr, gj = x0 - H + cc;
            unk[q] = gi >= 0 && gi < N && gj >= 0 && gj < N;
            if (unk[q]) bv[q] = sb[(int64_t)rr * P + cc];
        }
    }
    __syncthreads();
    uint32_t m = 0;
    if (check) {
#pragma unroll
        for (int q = 0; q < kPersistCellsPerThread; ++q) {
            const int rr = ra[q], cc = ca[q];
            if (rr >= H && rr < H + h && cc >= H && cc < H + w) {
                const int c = rr * lp + cc;
                const uint32_t v = residual_bits(A[c], A[c + 1], A[c - 1], A[c - lp], A[c + lp], bv[q], r);
                m = m > v ? m : v;
            }
        }
    }
    float* cur = A;
    float* nxt = B;
    for (int sw = 1; sw <= Dc; ++sw) {
        const int lo = a.async_mode ? 1 : sw;  // exact tiles shrink; async tiles keep their core
        const int hir = lh - lo, hic = lp - lo;
#pragma unroll
        for (int q = 0; q < kPersistCellsPerThread; ++q) {
            const int rr = ra[q], cc = ca[q];
            if (unk[q] && rr >= lo && rr < hir && cc >= lo && cc < hic) {
                const int c = rr * lp + cc;
                nxt[c] = jacobi_update<FAST>(cur[c + 1], cur[c - 1], cur[c - lp], cur[c + lp], bv[q], r, d, y);
            }
        }
        __syncthreads();
        float* t = cur;
        cur = nxt;
        nxt = t;
    }
    float* dst = uout + g.origin + (int64_t)(y0 - H) * P + (x0 - H);
#pragma unroll
    for (int q = 0; q < kPersistCellsPerThread; ++q) {
        const int rr = ra[q], cc = ca[q];
        if (rr >= H && rr < H + h && cc >= H && cc < H + w) dst[(int64_t)rr * P + cc] = cur[rr * lp + cc];
    }
    __syncthreads();  // the next tile re-stages the LDS buffers
    return m;
}

template <bool FAST>
__global__ __launch_bounds__(kPersistThreads) void k_persist(PersistArgs a) {
    extern __shared__ float lds[];
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int G = gridDim.x;
    const int ntiles = ((N + a.tx - 1) / a.tx) * ((N + a.ty - 1) / a.ty);
    const int ncol4 = (N + 3) / 4;
    int cur = a.cur0;
    int red = 0;        // reductions so far: selects the partial buffer
    uint32_t gen = 0;   // barrier generation
    for (int step = 0; step < a.nsteps; ++step) {
        // ---- b = u^n + s, partial max |b + r*g|
        {
            const float* u = cur ? a.u1 : a.u0;
            uint32_t m = 0;
            const int64_t total = (int64_t)N * ncol4;
            for (int64_t idx = (int64_t)blockIdx.x * kPersistThreads + threadIdx.x; idx < total;
                 idx += (int64_t)G * kPersistThreads) {
                const int i = (int)(idx / ncol4);
                const int j0 = (int)(idx - (int64_t)i * ncol4) * 4;
                const float rg = a.r * (i == 0 ? kTop : 0.0f);
                for (int c = 0; c < 4 && j0 + c < N; ++c) {
                    const int64_t o = g.origin + (int64_t)i * P + j0 + c;
                    const float bb = u[o] + a.s[o];
                    a.b[o] = bb;
                    const uint32_t v = __float_as_uint(fabsf(bb + rg));
                    m = m > v ? m : v;
                }
            }
            block_partial(m, a.partial, red & 1);
        }
        if (!grid_barrier(a.sc, gen)) return;
        const uint32_t bA_bits = reduce_partials(a.partial, red & 1);
        ++red;
        const float bA = __uint_as_float(bA_bits);
        int64_t k = 0;
        int done = 0;
        int status = 1;
        uint32_t R_bits = 0;
        for (;;) {
            const bool check = done == 0 && k > 0;
            const int left = a.L - done;
            const int Dc = a.D < left ? a.D : left;
            const float* uin = cur ? a.u1 : a.u0;
            float* uout = cur ? a.u0 : a.u1;
            uint32_t m = 0;
            for (int t = blockIdx.x; t < ntiles; t += G) {
                const uint32_t v = persist_tile<FAST>(a, uin, uout, t, Dc, check, lds);
                m = m > v ? m : v;
            }
            if (check) block_partial(m, a.partial, red & 1);
            if (!grid_barrier(a.sc, gen)) return;
            if (check) {
                R_bits = reduce_partials(a.partial, red & 1);
                ++red;
                const float rho = __uint_as_float(R_bits) / bA;
                if (!(rho >= a.tol)) {
                    status = (rho != rho) ? -5 : 0;  // JAC_ENAN : JAC_OK; the result is u_k
                    break;
                }
                if (k >= a.max_sweeps) {
                    status = -4;  // JAC_ENOCONV
                    break;
                }
            }
            cur ^= 1;
            k += Dc;
            done += Dc;
            if (done == a.L) done = 0;
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            PersistOut o;
            o.sweeps = k;
            o.R_bits = R_bits;
            o.bA_bits = bA_bits;
            o.status = status;
            o.cur = cur;
            a.out[step] = o;
        }
        if (status != 0) break;
    }
}

// ---------------------------------------------------------------- resident tiles
//
// The synchronous sweep (D = 1) on grids whose tiles all fit one round of
// co-resident blocks: each block owns one tile for the whole solve and keeps
// its two iterates (core plus a one-cell halo) and b in LDS, and s in
// registers.  After each sweep a block publishes the four edges of its new
// iterate and a flag; before the next sweep it waits for its (up to) four
// neighbours' flags and copies their edges into its halo.  A sweep then costs
// one point-to-point exchange instead of a re-staged tile and a grid-wide
// barrier; the norm of each step and each check's residual are grid-wide
// maxima of tagged words, again without a barrier (tagged_max).  Every block takes the same decisions from the same reduced values,
// so all sweep the same number of times; at a stop the result u_k is the
// block's current iterate, whose halo already holds the neighbours' u_k edges
// -- the next step starts from it without re-reading the grid.  The field is
// written back to memory when the solve ends (or a step fails).
//
// Exchange memory: the b plane (b lives in LDS here), per tile and parity 4
// edges of up to T cells -- top row, bottom row, left column, right column --
// each cell one 64-bit word: the value in the low half, the number of the
// sweep that produced it in the high half.  A writer stores each word with one
// coherent 64-bit store; a reader polls the word until its tag is the sweep it
// needs, then takes the value from the same word.  A 64-bit word is read and
// written whole, so no fence and no separate flag are needed.  Two parities:
// a block overwrites its sweep-s words with sweep s+2 only after it has read
// its neighbours' sweep-s+1 edges, which they publish only after reading its
// sweep-s ones.  The host clears the words before each solve.

constexpr int kResThreads = 1024;
constexpr int kResCellsPerThread = 4;  // core cells per thread: tiles of at most 64 x 64

__device__ __forceinline__ uint64_t* res_edges(uint64_t* xbuf, int tile, int parity, int T) {
    return xbuf + ((int64_t)tile * 2 + parity) * 4 * T;
}

// words of the edge exchange of a resident solve (cleared by the host)
int64_t resident_exchange_words(int ntiles, int T) { return (int64_t)ntiles * 8 * T; }

// Grid-wide max of `m` without a barrier: every block stores its block max
// tagged with the reduction number `serial` into its slot of buffer `which`
// (2 x gridDim.x 64-bit words, cleared by the host before the solve), then
// waits until every slot carries that tag and takes the max.  The same value
// in every block.  Two buffers: a block's next-but-one reduction can overwrite
// a slot only after every block has published the one in between, which each
// does only after reading this one.  Returns false (every block leaves) when a
// wait outlasts the spin budget or another block's did.
__device__ bool tagged_max(uint64_t* part, int which, uint32_t serial, uint32_t m, Scratch* sc, uint32_t* out) {
    __shared__ uint32_t wmax[kResThreads / 64];
    __shared__ uint32_t bad;
    const int G = gridDim.x;
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    uint64_t* slots = part + (int64_t)which * G;
    if (threadIdx.x == 0) {
        uint32_t r = wmax[0];
        for (int w = 1; w < kResThreads / 64; ++w) r = r > wmax[w] ? r : wmax[w];
        __hip_atomic_store(&slots[blockIdx.x], ((uint64_t)serial << 32) | r, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t v = 0;
    for (int i = threadIdx.x; i < G; i += kResThreads) {
        uint32_t spins = 0;
        uint64_t x;
        for (;;) {
            x = __hip_atomic_load(&slots[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(x >> 32) == serial) break;
            if ((++spins & 1023u) == 0u &&
                (__hip_atomic_load(&sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                 spins > kBarrierSpins)) {
                __hip_atomic_store(&sc->bar_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bad = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        const uint32_t xv = (uint32_t)x;
        v = v > xv ? v : xv;
    }
    __syncthreads();  // every thread is done with wmax before it is reused
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = wmax[0];
    for (int w = 1; w < kResThreads / 64; ++w) r = r > wmax[w] ? r : wmax[w];
    const bool ok = bad == 0;
    __syncthreads();
    *out = r;
    return ok;
}

template <bool FAST>
__global__ __launch_bounds__(kResThreads) void k_persist_res(PersistArgs a) {
    extern __shared__ float lds[];
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int T = a.tx;  // square tiles
    const int ntx = (N + T - 1) / T;
    const int tile = blockIdx.x;
    const int tx0 = (tile % ntx) * T, ty0 = (tile / ntx) * T;
    const int w = tx0 + T <= N ? T : N - tx0, h = ty0 + T <= N ? T : N - ty0;
    const int lp = w + 2, lh = h + 2;
    float* U[2] = {lds, lds + (T + 2) * (T + 2)};
    float* BL = lds + 2 * (T + 2) * (T + 2);
    uint64_t* xbuf = reinterpret_cast<uint64_t*>(a.b);  // edge exchange (see above)
    const float r = a.r, d = a.d, y = a.y;
    // neighbours: 0 north, 1 south, 2 west, 3 east (-1: none)
    const int nb_n = ty0 > 0 ? tile - ntx : -1, nb_s = ty0 + T < N ? tile + ntx : -1;
    const int nb_w = tx0 > 0 ? tile - 1 : -1, nb_e = tx0 + T < N ? tile + 1 : -1;

    // stage u^n with its halo (ghost ring included) into both buffers, s into registers
    {
        const float* src = (a.cur0 ? a.u1 : a.u0) + g.origin + (int64_t)(ty0 - 1) * P + (tx0 - 1);
        for (int k = threadIdx.x; k < lp * lh; k += kResThreads) {
            const int rr = k / lp, cc = k - rr * lp;
            const float v = src[(int64_t)rr * P + cc];
            U[0][rr * lp + cc] = v;
            U[1][rr * lp + cc] = v;
        }
    }
    float sv[kResCellsPerThread];
    int cell[kResCellsPerThread];  // LDS index of each core cell of this thread (-1: none)
#pragma unroll
    for (int q = 0; q < kResCellsPerThread; ++q) {
        const int k = threadIdx.x + q * kResThreads;
        cell[q] = -1;
        sv[q] = 0.0f;
        if (k < w * h) {
            const int i = k / w, j = k - i * w;
            cell[q] = (i + 1) * lp + (j + 1);
            sv[q] = a.s[g.origin + (int64_t)(ty0 + i) * P + (tx0 + j)];
        }
    }
    __syncthreads();
    int cur = 0;            // LDS buffer holding the current iterate
    int red = 0;            // reductions so far: selects the partial buffer, tags the next
    uint32_t serial = 0;    // sweeps published by this block in this solve
    uint32_t bA_bits = 0;
    uint64_t* part64 = reinterpret_cast<uint64_t*>(a.partial);  // 2 x grid tagged words
    int status = 1;
    for (int step = 0; step < a.nsteps; ++step) {
        // ---- b = u^n + s on the core, partial max |b + r*g|
        {
            uint32_t m = 0;
#pragma unroll
            for (int q = 0; q < kResCellsPerThread; ++q) {
                if (cell[q] < 0) continue;
                const int i = ty0 + (cell[q] / lp - 1);
                const float bb = U[cur][cell[q]] + sv[q];
                BL[cell[q]] = bb;
                const float rg = r * (i == 0 ? kTop : 0.0f);
                const uint32_t v = __float_as_uint(fabsf(bb + rg));
                m = m > v ? m : v;
            }
            if (!tagged_max(part64, red & 1, (uint32_t)red + 1u, m, a.sc, &bA_bits)) return;
            ++red;
        }
        const float bA = __uint_as_float(bA_bits);
        int64_t k = 0;
        uint32_t R_bits = 0;
        status = 1;
        for (;;) {
            if (k > 0 && k % a.L == 0) {
                // check: the residual of u_k on the core (the halo holds the neighbours' u_k)
                const float* A = U[cur];
                uint32_t m = 0;
#pragma unroll
                for (int q = 0; q < kResCellsPerThread; ++q) {
                    if (cell[q] < 0) continue;
                    const int c = cell[q];
                    const uint32_t v = residual_bits(A[c], A[c + 1], A[c - 1], A[c - lp], A[c + lp], BL[c], r);
                    m = m > v ? m : v;
                }
                if (!tagged_max(part64, red & 1, (uint32_t)red + 1u, m, a.sc, &R_bits)) return;
                ++red;
                const float rho = __uint_as_float(R_bits) / bA;
                if (!(rho >= a.tol)) {
                    status = (rho != rho) ? -5 : 0;  // JAC_ENAN : JAC_OK; the result is u_k
                    break;
                }
                if (k >= a.max_sweeps) {
                    status = -4;  // JAC_ENOCONV
                    break;
                }
            }
            // ---- one sweep of the core into the other buffer
            {
                const float* A = U[cur];
                float* Bn = U[cur ^ 1];
#pragma unroll
                for (int q = 0; q < kResCellsPerThread; ++q) {
                    if (cell[q] < 0) continue;
                    const int c = cell[q];
                    Bn[c] = jacobi_update<FAST>(A[c + 1], A[c - 1], A[c - lp], A[c + lp], BL[c], r, d, y);
                }
            }
            __syncthreads();
            cur ^= 1;
            ++k;
            ++serial;
            // ---- publish this tile's new edges, tagged with the sweep number
            {
                const float* A = U[cur];
                uint64_t* e = res_edges(xbuf, tile, serial & 1, T);
                const uint64_t tag = (uint64_t)serial << 32;
                for (int q = threadIdx.x; q < 2 * (w + h); q += kResThreads) {
                    float v;
                    int slot;
                    if (q < w) { v = A[1 * lp + 1 + q]; slot = q; }                                    // top row
                    else if (q < 2 * w) { v = A[h * lp + 1 + (q - w)]; slot = T + (q - w); }            // bottom row
                    else if (q < 2 * w + h) { v = A[(1 + q - 2 * w) * lp + 1]; slot = 2 * T + (q - 2 * w); }  // left
                    else { v = A[(1 + q - 2 * w - h) * lp + w]; slot = 3 * T + (q - 2 * w - h); }           // right
                    __hip_atomic_store(&e[slot], tag | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            // ---- take the neighbours' edges of this sweep into the halo:
            // north's bottom row -> halo row 0, south's top row -> row h+1,
            // west's right column -> column 0, east's left column -> column w+1
            {
                float* A = U[cur];
                for (int q = threadIdx.x; q < 2 * (w + h); q += kResThreads) {
                    int nbv, slot, dst;
                    if (q < w) { nbv = nb_n; slot = T + q; dst = 0 * lp + 1 + q; }
                    else if (q < 2 * w) { nbv = nb_s; slot = q - w; dst = (h + 1) * lp + 1 + (q - w); }
                    else if (q < 2 * w + h) { nbv = nb_w; slot = 3 * T + (q - 2 * w); dst = (1 + q - 2 * w) * lp; }
                    else { nbv = nb_e; slot = 2 * T + (q - 2 * w - h); dst = (1 + q - 2 * w - h) * lp + w + 1; }
                    if (nbv < 0) continue;  // a ghost cell: it keeps its fixed value
                    const uint64_t* src = res_edges(xbuf, nbv, serial & 1, T) + slot;
                    uint64_t x;
                    uint32_t spins = 0;
                    for (;;) {
                        x = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if ((uint32_t)(x >> 32) == serial) break;
                        if ((++spins & 1023u) == 0u &&
                            (__hip_atomic_load(&a.sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                             spins > kBarrierSpins)) {
                            __hip_atomic_store(&a.sc->bar_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    A[dst] = __uint_as_float((uint32_t)x);
                }
            }
            __syncthreads();
            if (__hip_atomic_load(&a.sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            PersistOut o;
            o.sweeps = k;
            o.R_bits = R_bits;
            o.bA_bits = bA_bits;
            o.status = status;
            o.cur = a.cur0;
            a.out[step] = o;
        }
        if (status != 0) break;
    }
    // the field: the core of the current iterate, into the buffer u^n came from
    {
        float* dst = (a.cur0 ? a.u1 : a.u0) + g.origin + (int64_t)ty0 * P + tx0;
#pragma unroll
        for (int q = 0; q < kResCellsPerThread; ++q) {
            if (cell[q] < 0) continue;
            const int i = cell[q] / lp - 1, j = cell[q] - (i + 1) * lp - 1;
            dst[(int64_t)i * P + j] = U[cur][cell[q]];
        }
    }
}

// Tile core for the exact tiles: large enough that staging and halo work stay
// moderate, small enough to give several blocks work on small grids.
static void persist_tiles(int N, int D, bool async_mode, int tile_x, int tile_y, int side, int* tx, int* ty) {
    if (async_mode) {
        *tx = tile_x;
        *ty = tile_y;
        return;
    }
    int t = side > 0 ? side : (N <= 384 ? 32 : 64);
    if ((t + 2 * D) * (t + 2 * D) > kPersistMaxCells) t = 90 - 2 * D;  // 90^2 <= 8192
    *tx = t;
    *ty = t;
}

struct PersistPlan {
    int tx, ty, grid, cells;
    size_t lds;
};

hipError_t persist_plan(int N, int D, bool async_mode, int tile_x, int tile_y, int side, bool fast, int cus,
                        PersistPlan* p) {
    persist_tiles(N, D, async_mode, tile_x, tile_y, side, &p->tx, &p->ty);
    const int H = async_mode ? 1 : D;
    p->cells = (p->tx + 2 * H) * (p->ty + 2 * H);
    if (p->cells > kPersistMaxCells) return hipErrorInvalidValue;
    p->lds = (size_t)2 * p->cells * sizeof(float);
    int per_cu = 0;
    hipError_t e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist<true>, kPersistThreads,
                                                                      p->lds)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist<false>,
                                                                      kPersistThreads, p->lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int64_t tiles = (int64_t)((N + p->tx - 1) / p->tx) * ((N + p->ty - 1) / p->ty);
    int64_t grid = (int64_t)cus * per_cu;
    if (tiles < grid) grid = tiles;
    if (grid > kMaxPersistBlocks) grid = kMaxPersistBlocks;
    p->grid = (int)grid;
    return hipSuccess;
}

hipError_t launch_persist(const StepArgs& sa, float* u0, float* u1, float* b, const float* s, uint32_t* partial,
                          void* out, int nsteps, int cur0, bool async_mode, int D, int L, int tile_x, int tile_y,
                          int side, int64_t max_sweeps, int cus, int* grid_used, hipStream_t stream) {
    PersistPlan p;
    hipError_t e = persist_plan(sa.g.N, D, async_mode, tile_x, tile_y, side, sa.fastdiv != 0, cus, &p);
    if (e != hipSuccess) return e;
    PersistArgs a;
    a.g = sa.g;
    a.r = sa.r;
    a.d = sa.d;
    a.y = sa.y;
    a.tol = sa.tol;
    a.u0 = u0;
    a.u1 = u1;
    a.b = b;
    a.s = s;
    a.partial = partial;
    a.out = reinterpret_cast<PersistOut*>(out);
    a.nsteps = nsteps;
    a.cur0 = cur0;
    a.async_mode = async_mode ? 1 : 0;
    a.D = D;
    a.L = L;
    a.tx = p.tx;
    a.ty = p.ty;
    a.lds_cells = p.cells;
    a.sc = sa.sc;
    a.max_sweeps = max_sweeps;
    // The synchronous sweep on a grid whose tiles all fit one round: resident
    // tiles (k_persist_res); otherwise re-staged tiles (k_persist).
    bool resident = false;
    int rgrid = 0, T = 0;
    size_t rlds = 0;
    if (!async_mode && D == 1) {
        T = side > 0 ? side : (sa.g.N <= 384 ? 32 : 64);
        const int64_t nt = (int64_t)((sa.g.N + T - 1) / T) * ((sa.g.N + T - 1) / T);
        rlds = (size_t)3 * (T + 2) * (T + 2) * sizeof(float);
        int per_cu = 0;
        if (T >= 1 && T * T <= kResThreads * kResCellsPerThread &&
            (sa.fastdiv ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_res<true>, kResThreads, rlds)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_res<false>, kResThreads,
                                                                       rlds)) == hipSuccess &&
            per_cu > 0 && nt <= (int64_t)cus * per_cu && nt <= kMaxPersistBlocks &&
            2 * resident_exchange_words((int)nt, T) <= sa.g.plane) {  // the edge exchange fits the b plane
            resident = true;
            rgrid = (int)nt;
        }
    }
    if (resident) {
        a.tx = a.ty = T;
        *grid_used = rgrid;
    } else {
        *grid_used = p.grid;
    }
    // clear the barrier words (release, error) and the grid's flag lines with kernel fills
    e = launch_fill(reinterpret_cast<float*>(&sa.sc->bar_release), 48, 0.0f, stream);
    if (e == hipSuccess)
        e = launch_fill(reinterpret_cast<float*>(scratch_flags(sa.sc)), (int64_t)(*grid_used) * kFlagStride, 0.0f,
                        stream);
    // tags of an earlier solve must not match: clear the exchange words
    if (e == hipSuccess && resident)
        e = launch_fill(b, 2 * resident_exchange_words(rgrid, T), 0.0f, stream);
    if (e == hipSuccess && resident)  // the 2 x grid tagged partial words
        e = launch_fill(reinterpret_cast<float*>(partial), 4 * (int64_t)rgrid, 0.0f, stream);
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    if (resident) {
        const void* fr = sa.fastdiv ? reinterpret_cast<const void*>(k_persist_res<true>)
                                    : reinterpret_cast<const void*>(k_persist_res<false>);
        return hipLaunchCooperativeKernel(fr, dim3(rgrid), dim3(kResThreads), args, (unsigned)rlds, stream);
    }
    const void* fn = sa.fastdiv ? reinterpret_cast<const void*>(k_persist<true>)
                                : reinterpret_cast<const void*>(k_persist<false>);
    return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kPersistThreads), args, (unsigned)p.lds, stream);
}

size_t persist_out_bytes() { return sizeof(PersistOut); }

}  // namespace jac
