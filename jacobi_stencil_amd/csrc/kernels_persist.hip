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
// Three kernels.  k_persist_res (below) keeps every tile resident in LDS for
// the whole solve and trades tile edges point to point; it serves SYNC and
// TBLOCK wherever all tiles fit one round of co-resident blocks, and
// k_persist_ares does the same for ASYNC.  k_persist re-stages tiles per chunk
// behind grid barriers and serves everything else.
//
// k_persist: every block runs the same program:
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
    uint32_t* partial;   // 2 x gridDim.x slots (double-buffered); resident tiles: 2 x gridDim.x 64-bit words
    uint64_t* xchg;      // resident tiles: the edge exchange (see below)
    PersistOut* out;     // nsteps records, pinned host memory
    int nsteps, cur0;
    int async_mode;      // 0: exact tiles (ghost zone), 1: block-asynchronous tiles
    int D, L;            // sweeps per chunk, check interval
    int tx, ty;          // tile core
    int group;           // resident block-asynchronous tiles: tiles per block
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
// The exact kernels (SYNC, TBLOCK) on grids whose tiles all fit one round of
// co-resident blocks: each block owns one square tile for the whole solve and
// keeps, in LDS, its region -- the tile plus a halo H = D + 1 cells deep -- as
// two iterates and s, with b of its cells in registers.  A chunk of Dc <= D
// sweeps updates the region's interior every sweep; after sweep t the cells at
// least t cells inside the region's edge are exact (the ghost-zone scheme of
// page "stencil-jacobian.vercel.app", section 02), so afterwards the core and
// the ring around it hold exactly Dc synchronous sweeps.  The ring lets the block measure the residual of its
// core at the end of a chunk without waiting for its neighbours.  The block
// then publishes the four H-deep strips along its core's edges, and the
// partial maximum of a check beside them, and refills its halo from its (up to)
// eight neighbours' strips; ghost cells (outside the grid) keep their fixed
// values.  A chunk costs one point-to-point exchange, and a check's grid-wide
// maximum completes under that same exchange -- no re-staged tile and no
// grid-wide barrier.  Every block takes the same decisions from the same
// reduced values; at a stop the result u_k is the block's current iterate,
// whose halo already holds the neighbours' u_k, so the next step starts from
// it without re-reading the grid.  The field goes back to memory when the
// solve ends (or a step fails).
//
// Exchange memory (the workspace's exchange region, cleared by the host before
// each solve): per tile and parity four strips of up to H x T cells -- top
// rows, bottom rows, left columns, right columns of the core -- each cell one
// 64-bit word, the value in the low half and the number of the chunk that
// produced it in the high half.  A writer stores each word with one coherent
// 64-bit store; a reader polls the word until its tag is the chunk it needs
// and takes the value from the same word, so no fence or flag is needed.  Two
// parities: a block overwrites its chunk-c words with chunk c+2 only after it
// has read its neighbours' chunk-c+1 strips, which they publish only after
// reading its chunk-c ones.  Tiles are at least H cells on each side, so every
// halo cell lies in one neighbour's strip.

constexpr int kResThreads = 1024;
constexpr int kResWaves = kResThreads / 64;
constexpr int kResCells = 9;   // interior cells per thread: (T + 2H - 2)^2 <= 9216
constexpr int kResPub = 5;     // strip words per thread: 4 H T <= 5120
constexpr int kResRef = 6;     // halo words per thread: 4 H T + 4 H^2 <= 6144
constexpr int kResPoll = 2;    // partial slots per thread: grid <= 2048

// words of the edge exchange of a resident solve with halo depth H
int64_t resident_exchange_words(int ntiles, int H, int T) { return (int64_t)ntiles * 8 * H * T; }

// Max over the 64 lanes of a wavefront with DPP moves (no LDS round trips):
// within each quad, across the quads of a 16-lane row (row rotations), then
// across rows (row broadcasts of lanes 15 and 31); lane 63 ends with the max.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xb1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4e, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xf, 0xf, false));  // row_ror 4
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xf, 0xf, false));  // row_ror 8
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast 15
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast 31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Block max of one value per thread through `wmax` (kResWaves words of LDS);
// the caller places the barrier between the two halves.
__device__ __forceinline__ void block_max_put(uint32_t* wmax, uint32_t v) {
    v = wave_max_dpp(v);
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = v;
}
__device__ __forceinline__ uint32_t block_max_get(const uint32_t* wmax) {
    uint32_t r = wmax[0];
#pragma unroll
    for (int w = 1; w < kResWaves; ++w) r = r > wmax[w] ? r : wmax[w];
    return r;
}

// Polls two groups of tagged 64-bit words -- n1 at base1 + off1[q] that must
// carry tag1, n2 at base2 + off2[q] that must carry tag2 (offset -1: none) --
// with every load of a round in flight at once, until each carries its tag.
// Returns false when the wait outlasts the spin budget or another block gave
// up (the error word), after setting that word.
template <int n1, int n2>
__device__ __forceinline__ bool poll_tagged(const uint64_t* base1, const int* off1, uint32_t tag1, uint64_t* x1,
                                            const uint64_t* base2, const int* off2, uint32_t tag2, uint64_t* x2,
                                            Scratch* sc) {
#pragma unroll
    for (int q = 0; q < n1; ++q)
        x1[q] = off1[q] >= 0 ? __hip_atomic_load(&base1[off1[q]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : ((uint64_t)tag1 << 32);
#pragma unroll
    for (int q = 0; q < n2; ++q)
        x2[q] = off2[q] >= 0 ? __hip_atomic_load(&base2[off2[q]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : ((uint64_t)tag2 << 32);
    uint32_t spins = 0;
    for (;;) {
        bool pending = false;
#pragma unroll
        for (int q = 0; q < n1; ++q) pending |= (uint32_t)(x1[q] >> 32) != tag1;
#pragma unroll
        for (int q = 0; q < n2; ++q) pending |= (uint32_t)(x2[q] >> 32) != tag2;
        if (!pending) return true;
        if ((++spins & 1023u) == 0u &&
            (__hip_atomic_load(&sc->bar_error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
             spins > kBarrierSpins)) {
            __hip_atomic_store(&sc->bar_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int q = 0; q < n1; ++q)
            if ((uint32_t)(x1[q] >> 32) != tag1)
                x1[q] = __hip_atomic_load(&base1[off1[q]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 0; q < n2; ++q)
            if ((uint32_t)(x2[q] >> 32) != tag2)
                x2[q] = __hip_atomic_load(&base2[off2[q]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Per-cell bits of the resident kernel: an unknown (a grid point), in the
// core, in the grid's top row.
constexpr uint32_t kCellUnk = 1u, kCellCore = 2u, kCellTop = 4u;

// LDS word at a byte offset (the neighbour offsets below fold into the
// instructions' immediate fields).
__device__ __forceinline__ float& lds_at(float* lds, int byte) {
    return *reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + byte);
}

// One sweep over this thread's NQ cells of the region's interior (every cell
// but the outermost ring), without branches.  `at[q]` is the byte offset of
// the cell's west neighbour in buffer 0; `oa` and `ob` are the byte offsets of
// the source and target buffers, lp4 the region pitch in bytes.  Every cell is
// updated every sweep; a cell fewer than `sw` cells inside the region's edge
// gets a value nothing reads before the halo refill overwrites it (the exact
// cells lie ever deeper inside), so only the grid's fixed cells are masked.
template <bool FAST, int NQ>
__device__ __forceinline__ void res_sweep(float* lds, int oa, int ob, int lp4, const int* at, const uint32_t* info,
                                          const float* bv, float r, float d, float y) {
#pragma unroll
    for (int g0 = 0; g0 < NQ; g0 += 4) {  // four cells at a time: all loads, then all stores
        constexpr int kG = 4;
        float v[kG];
#pragma unroll
        for (int q = g0; q < (g0 + kG < NQ ? g0 + kG : NQ); ++q) {
            const int w = at[q] + oa;
            v[q - g0] = jacobi_update<FAST>(lds_at(lds, w + 8), lds_at(lds, w), lds_at(lds, w - lp4 + 4),
                                            lds_at(lds, w + lp4 + 4), bv[q], r, d, y);
        }
#pragma unroll
        for (int q = g0; q < (g0 + kG < NQ ? g0 + kG : NQ); ++q)
            if (info[q] & kCellUnk) lds_at(lds, at[q] + ob + 4) = v[q - g0];
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Dc sweeps, buffers alternating from `cur` (R floats apart); returns the
// buffer that holds the last sweep.
template <bool FAST, int NQ>
__device__ __forceinline__ int res_sweeps(float* lds, int cur, int Dc, int R, int lp4, const int* at,
                                          const uint32_t* info, const float* bv, float r, float d, float y) {
    for (int sw = 1; sw <= Dc; ++sw) {
        res_sweep<FAST, NQ>(lds, cur * R * 4, (cur ^ 1) * R * 4, lp4, at, info, bv, r, d, y);
        __syncthreads();
        cur ^= 1;
    }
    return cur;
}

// The residual bits max over this thread's core cells (buffer at byte offset oa).
template <int NQ>
__device__ __forceinline__ uint32_t res_check(float* lds, int oa, int lp4, const int* at, const uint32_t* info,
                                              const float* bv, float r) {
    uint32_t m = 0;
#pragma unroll
    for (int g0 = 0; g0 < NQ; g0 += 4) {
#pragma unroll
        for (int q = g0; q < (g0 + 4 < NQ ? g0 + 4 : NQ); ++q) {
            const int w = at[q] + oa;
            const uint32_t v = residual_bits(lds_at(lds, w + 4), lds_at(lds, w + 8), lds_at(lds, w),
                                             lds_at(lds, w - lp4 + 4), lds_at(lds, w + lp4 + 4), bv[q], r);
            m = (info[q] & kCellCore) && v > m ? v : m;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return m;
}

#define JAC_RES_NQ(CALL)                 \
    switch (nq) {                        \
        case 1: CALL(1); break;          \
        case 2: CALL(2); break;          \
        case 3: CALL(3); break;          \
        case 4: CALL(4); break;          \
        case 5: CALL(5); break;          \
        case 6: CALL(6); break;          \
        case 7: CALL(7); break;          \
        case 8: CALL(8); break;          \
        default: CALL(9); break;         \
    }

template <bool FAST>
__global__ __launch_bounds__(kResThreads) void k_persist_res(PersistArgs a) {
    extern __shared__ float lds[];
    __shared__ uint32_t wmax[kResWaves];
    __shared__ uint32_t gave_up;  // a wait of this block outlasted the spin budget
    __shared__ int nbase[8];      // exchange offset of each neighbour's strips (N S W E NW NE SW SE)
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int T = a.tx, H = a.D + 1;  // square tiles; halo one deeper than a chunk
    const int ntx = (N + T - 1) / T;
    const int tile = blockIdx.x;
    const int ti = tile / ntx, tj = tile % ntx;
    const int tx0 = tj * T, ty0 = ti * T;
    const int w = tx0 + T <= N ? T : N - tx0, h = ty0 + T <= N ? T : N - ty0;
    const int lp = w + 2 * H, lh = h + 2 * H;  // region pitch and height
    // LDS: iterates at [0, R) and [R, 2R), s at [2R, 3R), the dummy word at 3R
    const int R = (T + 2 * H) * (T + 2 * H), dummy = 3 * R;
    const float r = a.r, d = a.d, y = a.y;
    const int tid = threadIdx.x;
    if (tid == 0) gave_up = 0;

    // the region of u^n (ghost ring and padding included) into both buffers,
    // s of its unknowns beside them
    {
        const float* src = (a.cur0 ? a.u1 : a.u0) + g.origin + (int64_t)(ty0 - H) * P + (tx0 - H);
        for (int k = tid; k < lp * lh; k += kResThreads) {
            const int rr = k / lp, cc = k - rr * lp;
            const int gi = ty0 - H + rr, gj = tx0 - H + cc;
            const float v = src[(int64_t)rr * P + cc];
            lds[k] = v;
            lds[R + k] = v;
            lds[2 * R + k] = (gi >= 0 && gi < N && gj >= 0 && gj < N) ? a.s[g.origin + (int64_t)gi * P + gj] : 0.0f;
        }
    }
    // this thread's cells of the region's interior (inner cell k = tid +
    // q*kResThreads, row 1 + k / (lp-2), column 1 + k % (lp-2)): the byte offset
    // of its west neighbour and its bits; a lane past the interior keeps an
    // interior cell's offset and no bits
    const int nin = (lp - 2) * (lh - 2);
    const int nq = (nin + kResThreads - 1) / kResThreads;
    int at[kResCells];
    uint32_t info[kResCells];
#pragma unroll
    for (int q = 0; q < kResCells; ++q) {
        const int k = tid + q * kResThreads;
        const int kk = k < nin ? k : 0;
        const int rr = 1 + kk / (lp - 2), cc = 1 + kk % (lp - 2);
        const int gi = ty0 - H + rr, gj = tx0 - H + cc;
        at[q] = (rr * lp + cc - 1) * 4;
        info[q] = 0;
        if (k < nin && gi >= 0 && gi < N && gj >= 0 && gj < N) {
            info[q] = kCellUnk;
            if (rr >= H && rr < H + h && cc >= H && cc < H + w) info[q] |= kCellCore;
            if (gi == 0) info[q] |= kCellTop;
        }
    }
    // the exchange maps in LDS: per strip word this block publishes, LDS cell
    // << 16 | slot; per halo word it takes, neighbour << 27 | slot << 14 | LDS
    // cell (all ones: a ghost cell)
    const int HT = H * T;
    const int npub = 2 * H * w + 2 * h * H, nref = npub + 4 * H * H;
    uint32_t* pubmap = reinterpret_cast<uint32_t*>(lds + dummy + 1);
    uint32_t* refmap = pubmap + 4 * HT;
    if (tid < 8) {
        const int di = (tid == 0 || tid == 4 || tid == 5) ? -1 : (tid == 1 || tid == 6 || tid == 7) ? 1 : 0;
        const int dj = (tid == 2 || tid == 4 || tid == 6) ? -1 : (tid == 3 || tid == 5 || tid == 7) ? 1 : 0;
        nbase[tid] = ((ti + di) * ntx + (tj + dj)) * 8 * HT;  // used only where that neighbour exists
    }
    {
        const int nrow = H * w, ncol = h * H;
        for (int q = tid; q < npub; q += kResThreads) {
            int src, slot;
            if (q < nrow) {  // top H rows of the core
                const int i = q / w, j = q - i * w;
                src = (H + i) * lp + H + j;
                slot = i * T + j;
            } else if (q < 2 * nrow) {  // bottom H rows
                const int qq = q - nrow, i = qq / w, j = qq - i * w;
                src = (h + i) * lp + H + j;
                slot = HT + i * T + j;
            } else if (q < 2 * nrow + ncol) {  // left H columns
                const int qq = q - 2 * nrow, i = qq / H, j = qq - i * H;
                src = (H + i) * lp + H + j;
                slot = 2 * HT + i * H + j;
            } else {  // right H columns
                const int qq = q - 2 * nrow - ncol, i = qq / H, j = qq - i * H;
                src = (H + i) * lp + w + j;
                slot = 3 * HT + i * H + j;
            }
            pubmap[q] = ((uint32_t)src << 16) | (uint32_t)slot;
        }
        const int ncor = H * H;
        auto has = [&](int di, int dj) {
            const int i = ti + di, j = tj + dj;
            return i >= 0 && i < ntx && j >= 0 && j < ntx;
        };
        for (int q = tid; q < nref; q += kResThreads) {
            int dir, slot, dst;
            bool ok;
            if (q < nrow) {  // north neighbour's bottom rows -> halo rows 0..H-1
                const int i = q / w, j = q - i * w;
                dir = 0; ok = has(-1, 0); slot = HT + i * T + j; dst = i * lp + H + j;
            } else if (q < 2 * nrow) {  // south's top rows -> rows H+h..
                const int qq = q - nrow, i = qq / w, j = qq - i * w;
                dir = 1; ok = has(1, 0); slot = i * T + j; dst = (H + h + i) * lp + H + j;
            } else if (q < 2 * nrow + ncol) {  // west's right columns -> columns 0..H-1
                const int qq = q - 2 * nrow, i = qq / H, j = qq - i * H;
                dir = 2; ok = has(0, -1); slot = 3 * HT + i * H + j; dst = (H + i) * lp + j;
            } else if (q < 2 * nrow + 2 * ncol) {  // east's left columns -> columns H+w..
                const int qq = q - 2 * nrow - ncol, i = qq / H, j = qq - i * H;
                dir = 3; ok = has(0, 1); slot = 2 * HT + i * H + j; dst = (H + i) * lp + H + w + j;
            } else {  // corners: the diagonal neighbours' bottom / top rows
                const int qq = q - 2 * nrow - 2 * ncol, c4 = qq / ncor, i = (qq - c4 * ncor) / H,
                          j = qq - c4 * ncor - i * H;
                dir = 4 + c4;
                if (c4 == 0) {         // north-west: bottom rows, last H columns (a full-width tile)
                    ok = has(-1, -1); slot = HT + i * T + (T - H + j); dst = i * lp + j;
                } else if (c4 == 1) {  // north-east: bottom rows, first H columns
                    ok = has(-1, 1); slot = HT + i * T + j; dst = i * lp + H + w + j;
                } else if (c4 == 2) {  // south-west: top rows, last H columns
                    ok = has(1, -1); slot = i * T + (T - H + j); dst = (H + h + i) * lp + j;
                } else {               // south-east: top rows, first H columns
                    ok = has(1, 1); slot = i * T + j; dst = (H + h + i) * lp + H + w + j;
                }
            }
            refmap[q] = ok ? ((uint32_t)dir << 27) | ((uint32_t)slot << 14) | (uint32_t)dst : 0xFFFFFFFFu;
        }
    }
    __syncthreads();
    uint64_t* xbuf = a.xchg;
    uint64_t* part64 = reinterpret_cast<uint64_t*>(a.partial);  // 2 x grid tagged words
    const int G = gridDim.x;
    int cur = 0;            // LDS buffer holding the current iterate
    int red = 0;            // reductions so far: selects the partial buffer, tags the next
    uint32_t serial = 0;    // chunks published by this block in this solve
    uint32_t bA_bits = 0;
    int status = 1;
    float bv[kResCells];    // b of this thread's cells
    for (int step = 0; step < a.nsteps; ++step) {
        // ---- b = u^n + s on the region's unknowns, max |b + r*g| on the core
        {
            __syncthreads();  // every thread has read the last reduction from wmax
            const int ob4 = cur * R * 4;
            uint32_t m = 0;
#pragma unroll
            for (int q = 0; q < kResCells; ++q) {
                bv[q] = 0.0f;
                if (!(info[q] & kCellUnk)) continue;
                bv[q] = lds_at(lds, at[q] + ob4 + 4) + lds_at(lds, at[q] + 2 * R * 4 + 4);
                if (info[q] & kCellCore) {
                    float tg = kTop;
                    asm volatile("" : "+v"(tg));
                    const float rg = r * ((info[q] & kCellTop) ? tg : 0.0f);
                    const uint32_t v = __float_as_uint(fabsf(bv[q] + rg));
                    m = m > v ? m : v;
                }
            }
            block_max_put(wmax, m);
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&part64[(int64_t)(red & 1) * G + blockIdx.x],
                                   ((uint64_t)(red + 1) << 32) | block_max_get(wmax), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            int off[kResPoll];
            uint64_t x[kResPoll];
#pragma unroll
            for (int q = 0; q < kResPoll; ++q) {
                const int i = tid + q * kResThreads;
                off[q] = i < G ? (red & 1) * G + i : -1;
            }
            if (!poll_tagged<0, kResPoll>(nullptr, nullptr, 0u, nullptr, part64, off, (uint32_t)red + 1u, x, a.sc))
                gave_up = 1;
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < kResPoll; ++q) v = off[q] >= 0 && (uint32_t)x[q] > v ? (uint32_t)x[q] : v;
            __syncthreads();  // wmax read by thread 0 above
            block_max_put(wmax, v);
            __syncthreads();
            bA_bits = block_max_get(wmax);
            if (gave_up) return;
            ++red;
        }
        const float bA = __uint_as_float(bA_bits);
        int64_t k = 0;
        int done = 0;
        uint32_t R_bits = 0;
        status = 1;
        for (;;) {
            const int left = a.L - done;
            const int Dc = a.D < left ? a.D : left;
            // ---- Dc sweeps; the exact region shrinks by a cell per sweep
#define JAC_RES_SWEEPS(NQ) cur = res_sweeps<FAST, NQ>(lds, cur, Dc, R, lp * 4, at, info, bv, r, d, y)
            JAC_RES_NQ(JAC_RES_SWEEPS)
#undef JAC_RES_SWEEPS
            k += Dc;
            done += Dc;
            if (done == a.L) done = 0;
            ++serial;
            const int ob = cur * R;
            const bool check = done == 0;
            // ---- publish the core's H-deep edge strips, tagged with the chunk number
            {
                uint64_t* e = xbuf + ((int64_t)tile * 2 + (serial & 1)) * 4 * HT;
                const uint64_t tag = (uint64_t)serial << 32;
#pragma unroll
                for (int q = 0; q < kResPub; ++q) {
                    const int i = tid + q * kResThreads;
                    if (i >= npub) break;
                    const uint32_t m = pubmap[i];
                    __hip_atomic_store(&e[m & 0xFFFFu], tag | __float_as_uint(lds[ob + (int)(m >> 16)]),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            // ---- a check: the residual of u_k on the core (its ring is exact);
            // the block's partial goes out before the halo wait
            if (check) {
                uint32_t m = 0;
#define JAC_RES_CHECK(NQ) m = res_check<NQ>(lds, ob * 4, lp * 4, at, info, bv, r)
                JAC_RES_NQ(JAC_RES_CHECK)
#undef JAC_RES_CHECK
                block_max_put(wmax, m);
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(&part64[(int64_t)(red & 1) * G + blockIdx.x],
                                       ((uint64_t)(red + 1) << 32) | block_max_get(wmax), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            // ---- refill the halo from the neighbours' strips of this chunk, and
            // at a check take every block's partial: all words in flight at once
            uint32_t pv = 0;
            {
                const int par = (int)(serial & 1) * 4 * HT;
                int off1[kResRef], off2[kResPoll], dst1[kResRef];
                uint64_t x1[kResRef], x2[kResPoll];
#pragma unroll
                for (int q = 0; q < kResRef; ++q) {
                    const int i = tid + q * kResThreads;
                    const uint32_t m = i < nref ? refmap[i] : 0xFFFFFFFFu;
                    off1[q] = m == 0xFFFFFFFFu ? -1 : nbase[m >> 27] + par + (int)((m >> 14) & 8191u);
                    dst1[q] = m == 0xFFFFFFFFu ? dummy : ob + (int)(m & 16383u);
                }
#pragma unroll
                for (int q = 0; q < kResPoll; ++q) {
                    const int i = tid + q * kResThreads;
                    off2[q] = check && i < G ? (red & 1) * G + i : -1;
                }
                if (!poll_tagged<kResRef, kResPoll>(xbuf, off1, serial, x1, part64, off2, (uint32_t)red + 1u, x2,
                                                    a.sc))
                    gave_up = 1;
#pragma unroll
                for (int q = 0; q < kResRef; ++q)
                    lds[dst1[q]] = __uint_as_float((uint32_t)x1[q]);
#pragma unroll
                for (int q = 0; q < kResPoll; ++q) pv = off2[q] >= 0 && (uint32_t)x2[q] > pv ? (uint32_t)x2[q] : pv;
            }
            if (check) {
                __syncthreads();  // thread 0 has read wmax
                block_max_put(wmax, pv);
            }
            __syncthreads();
            if (gave_up) return;
            if (check) {
                R_bits = block_max_get(wmax);
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
        const int ob = cur * R;
        for (int k = tid; k < w * h; k += kResThreads) {
            const int i = k / w, j = k - i * w;
            dst[(int64_t)i * P + j] = lds[ob + (H + i) * lp + H + j];
        }
    }
}

// ---------------------------------------------------------------- resident block-asynchronous tiles
//
// The block-asynchronous kernel (ASYNC) on grids whose tiles all fit one round
// of co-resident blocks: each block owns a group of G consecutive tx x ty
// tiles (in row-major tile order; G = 1 on small grids) and keeps three copies
// of each, with a one-cell halo, in LDS, and b of its cells in registers.  A
// chunk of Dc sweeps updates every tile with its halo frozen -- exactly one
// block-asynchronous launch (page "stencil-jacobian.vercel.app", section 02):
// tiles of one block see each other only through the halo refill, as tiles of
// different blocks do -- and writes only the two copies other than its input,
// so the chunk's input survives it.  Each tile then publishes its four edges
// and refills its halo from its neighbours' edges (no corners: the five-point
// stencil never reads them), in the tagged-word exchange described above, here
// one cell deep.  A check at k = gL (g >= 1) measures the residual of u_k once
// the halo holds the neighbours' u_k, as the re-staged kernel measures it at
// the start of the next chunk; the grid-wide maximum completes under the next
// chunk's exchange, and a stop keeps u_k, that chunk's preserved input, whose
// halo the dropped refill has left as it was.
//
// Exchange memory: per tile and parity 2 (tx + ty) words -- the top row
// [0, tx), the bottom row [tx, 2tx), the left column [2tx, 2tx + ty), the
// right column [2tx + ty, 2tx + 2ty) of the tile.  Tiles in one column share
// a width and tiles in one row a height, so every halo cell lies in one
// neighbour's edge, whatever the ragged last tiles.
//
// LDS: copy c of tile q of the group at floats (c G + q) R, R = (tx+2)(ty+2);
// the tile's cells at rows 1..h, columns 1..w of its copy (pitch tx + 2).

constexpr int kAresEdge = 2;  // edge words published and taken per thread: G (tx + ty) <= block size
constexpr int kAresPoll = 4;  // partial slots per thread: grid <= 4 x block size

int64_t ares_exchange_words(int ntiles, int tx, int ty) { return (int64_t)ntiles * 4 * (tx + ty); }

// Dc sweeps from copy `in` (copies RB floats apart) through the other two
// copies; returns the copy that holds the last sweep.
template <bool FAST, int NQ>
__device__ __forceinline__ int ares_sweeps(float* lds, int in, int Dc, int RB, int lp4, const int* at,
                                           const uint32_t* info, const float* bv, float r, float d, float y) {
    const int x = in == 2 ? 0 : in + 1, z = 3 - in - x;
    int src = in, dst = x;
    for (int sw = 1; sw <= Dc; ++sw) {
        res_sweep<FAST, NQ>(lds, src * RB * 4, dst * RB * 4, lp4, at, info, bv, r, d, y);
        __syncthreads();
        src = dst;
        dst = dst == x ? z : x;
    }
    return src;
}

// Geometry of tile t of a tx x ty tiling of the N x N grid.
struct AresTile {
    int ti, tj, x0, y0, w, h;
};
__device__ __forceinline__ AresTile ares_tile(int t, int N, int TX, int TY, int ntx) {
    AresTile g;
    g.ti = t / ntx;
    g.tj = t - g.ti * ntx;
    g.x0 = g.tj * TX;
    g.y0 = g.ti * TY;
    g.w = g.x0 + TX <= N ? TX : N - g.x0;
    g.h = g.y0 + TY <= N ? TY : N - g.y0;
    return g;
}

template <bool FAST>
__global__ __launch_bounds__(kResThreads) void k_persist_ares(PersistArgs a) {
    extern __shared__ float lds[];
    __shared__ uint32_t wmax[kResWaves];
    __shared__ uint32_t gave_up;  // a wait of this block outlasted the spin budget
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int TX = a.tx, TY = a.ty, GT = a.group;
    const int ntx = (N + TX - 1) / TX, nty = (N + TY - 1) / TY;
    const int t0 = blockIdx.x * GT;                                    // the group's first tile
    const int ng = ntx * nty - t0 < GT ? ntx * nty - t0 : GT;         // tiles in this group
    const int lp = TX + 2;            // copy pitch
    const int R = lp * (TY + 2);      // floats per tile copy
    const int RB = GT * R;            // floats per copy of the group
    const int TC = TX * TY;           // cell slots per tile
    const int EW = 2 * (TX + TY);     // exchange words per tile and parity
    const float r = a.r, d = a.d, y = a.y;
    const int tid = threadIdx.x, nthr = blockDim.x;
    if (tid < kResWaves) wmax[tid] = 0;  // the words of absent waves stay 0
    if (tid == 0) gave_up = 0;
    // each tile and its halo of u^n (ghost cells included) into all three copies
    for (int q = 0; q < ng; ++q) {
        const AresTile T = ares_tile(t0 + q, N, TX, TY, ntx);
        const float* src = (a.cur0 ? a.u1 : a.u0) + g.origin + (int64_t)(T.y0 - 1) * P + (T.x0 - 1);
        const int rw = T.w + 2;
        for (int k = tid; k < rw * (T.h + 2); k += nthr) {
            const int rr = k / rw, cc = k - rr * rw;
            const float v = src[(int64_t)rr * P + cc];
            const int c = q * R + rr * lp + cc;
            lds[c] = v;
            lds[RB + c] = v;
            lds[2 * RB + c] = v;
        }
    }
    // this thread's cells k = tid + n*nthr: tile k / TC of the group, cell
    // k % TC of it (row / w, column % w); the byte offset of the west
    // neighbour in copy 0 and the cell's bits; a lane past the cells keeps
    // cell 0's offset and no bits
    const int nq = (ng * TC + nthr - 1) / nthr;
    int at[kResCells];
    uint32_t info[kResCells];
#pragma unroll
    for (int n = 0; n < kResCells; ++n) {
        const int k = tid + n * nthr;
        const int q = k / TC, l = k - q * TC;
        at[n] = lp * 4;
        info[n] = 0u;
        if (q < ng) {
            const AresTile T = ares_tile(t0 + q, N, TX, TY, ntx);
            if (l < T.w * T.h) {
                const int i = l / T.w, j = l - i * T.w;
                at[n] = (q * R + (1 + i) * lp + j) * 4;
                info[n] = kCellUnk | kCellCore | (T.y0 + i == 0 ? kCellTop : 0u);
            }
        }
    }
    // the edge words this thread publishes (LDS cell, word without parity)
    // and takes (neighbour word without parity, LDS cell; -1: none or a ghost)
    int psrc[kAresEdge], pword[kAresEdge], roff[kAresEdge], rdst[kAresEdge];
#pragma unroll
    for (int p = 0; p < kAresEdge; ++p) {
        const int e = tid + p * nthr;
        const int q = e / EW, le = e - q * EW;
        psrc[p] = -1;
        pword[p] = 0;
        roff[p] = -1;
        rdst[p] = 0;
        if (q >= ng) continue;
        const AresTile T = ares_tile(t0 + q, N, TX, TY, ntx);
        const int w = T.w, h = T.h, ti = T.ti, tj = T.tj, base = q * R;
        int nb = -1, slot = 0;
        if (le < w) {  // top row; the halo row above from the north tile's bottom row
            psrc[p] = base + lp + 1 + le;
            slot = le;
            if (ti > 0) nb = (ti - 1) * ntx + tj, roff[p] = TX + le, rdst[p] = base + 1 + le;
        } else if (le < 2 * w) {  // bottom row; the halo row below from the south tile's top row
            const int jj = le - w;
            psrc[p] = base + h * lp + 1 + jj;
            slot = TX + jj;
            if (ti + 1 < nty) nb = (ti + 1) * ntx + tj, roff[p] = jj, rdst[p] = base + (h + 1) * lp + 1 + jj;
        } else if (le < 2 * w + h) {  // left column; the halo column left from the west tile's right column
            const int ii = le - 2 * w;
            psrc[p] = base + (1 + ii) * lp + 1;
            slot = 2 * TX + ii;
            if (tj > 0) nb = ti * ntx + tj - 1, roff[p] = 2 * TX + TY + ii, rdst[p] = base + (1 + ii) * lp;
        } else if (le < 2 * w + 2 * h) {  // right column; the halo column right from the east tile's left column
            const int ii = le - 2 * w - h;
            psrc[p] = base + (1 + ii) * lp + w;
            slot = 2 * TX + TY + ii;
            if (tj + 1 < ntx) nb = ti * ntx + tj + 1, roff[p] = 2 * TX + ii, rdst[p] = base + (1 + ii) * lp + w + 1;
        }
        pword[p] = (t0 + q) * 2 * EW + slot;
        if (nb >= 0) roff[p] += nb * 2 * EW;
    }
    __syncthreads();
    uint64_t* xbuf = a.xchg;
    uint64_t* part64 = reinterpret_cast<uint64_t*>(a.partial);  // 2 x grid tagged words
    const int G = gridDim.x;
    int cur = 0;            // copy holding the current iterate
    int red = 0;            // reductions so far: selects the partial buffer, tags the next
    uint32_t serial = 0;    // chunks published by this block in this solve
    uint32_t bA_bits = 0;
    int status = 1;
    float bv[kResCells];    // b of this thread's cells
    for (int step = 0; step < a.nsteps; ++step) {
        // ---- b = u^n + s on the tiles, max |b + r*g|
        {
            __syncthreads();  // every thread has read the last reduction from wmax
            const int ob4 = cur * RB * 4;
            uint32_t m = 0;
#pragma unroll
            for (int n = 0; n < kResCells; ++n) {
                bv[n] = 0.0f;
                if (!(info[n] & kCellUnk)) continue;
                const int k = tid + n * nthr, q = k / TC, l = k - q * TC;
                const AresTile T = ares_tile(t0 + q, N, TX, TY, ntx);
                const int i = l / T.w, j = l - i * T.w;
                bv[n] = lds_at(lds, at[n] + ob4 + 4) + a.s[g.origin + (int64_t)(T.y0 + i) * P + T.x0 + j];
                float tg = kTop;
                asm volatile("" : "+v"(tg));
                const float rg = r * ((info[n] & kCellTop) ? tg : 0.0f);
                const uint32_t v = __float_as_uint(fabsf(bv[n] + rg));
                m = m > v ? m : v;
            }
            block_max_put(wmax, m);
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&part64[(int64_t)(red & 1) * G + blockIdx.x],
                                   ((uint64_t)(red + 1) << 32) | block_max_get(wmax), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            int off[kAresPoll];
            uint64_t x[kAresPoll];
#pragma unroll
            for (int q = 0; q < kAresPoll; ++q) {
                const int i = tid + q * nthr;
                off[q] = i < G ? (red & 1) * G + i : -1;
            }
            if (!poll_tagged<0, kAresPoll>(nullptr, nullptr, 0u, nullptr, part64, off, (uint32_t)red + 1u, x, a.sc))
                gave_up = 1;
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < kAresPoll; ++q) v = off[q] >= 0 && (uint32_t)x[q] > v ? (uint32_t)x[q] : v;
            __syncthreads();  // wmax read by thread 0 above
            block_max_put(wmax, v);
            __syncthreads();
            bA_bits = block_max_get(wmax);
            if (gave_up) return;
            ++red;
        }
        const float bA = __uint_as_float(bA_bits);
        int64_t k = 0, kc = 0;  // sweeps; the pending check's sweep count
        int done = 0;
        bool pending = false;   // a check's partial is out; its decision comes with this chunk's exchange
        uint32_t R_bits = 0;
        status = 1;
        for (;;) {
            const int left = a.L - done;
            const int Dc = a.D < left ? a.D : left;
            const int in = cur;
            // ---- Dc sweeps with the halos frozen, into the copies other than `in`
#define JAC_ARES_SWEEPS(NQ) cur = ares_sweeps<FAST, NQ>(lds, in, Dc, RB, lp * 4, at, info, bv, r, d, y)
            JAC_RES_NQ(JAC_ARES_SWEEPS)
#undef JAC_ARES_SWEEPS
            k += Dc;
            done += Dc;
            if (done == a.L) done = 0;
            ++serial;
            const int ob = cur * RB;
            // ---- publish the tiles' edges, tagged with the chunk number
            {
                const int par = (int)(serial & 1) * EW;
                const uint64_t tag = (uint64_t)serial << 32;
#pragma unroll
                for (int p = 0; p < kAresEdge; ++p)
                    if (psrc[p] >= 0)
                        __hip_atomic_store(&xbuf[pword[p] + par], tag | __float_as_uint(lds[ob + psrc[p]]),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // ---- the neighbours' edges of this chunk, and with a pending check
            // every block's partial: all words in flight at once
            uint64_t x1[kAresEdge];
            uint32_t pv = 0;
            {
                const int par = (int)(serial & 1) * EW;
                int off1[kAresEdge], off2[kAresPoll];
                uint64_t x2[kAresPoll];
#pragma unroll
                for (int p = 0; p < kAresEdge; ++p) off1[p] = roff[p] >= 0 ? roff[p] + par : -1;
#pragma unroll
                for (int q = 0; q < kAresPoll; ++q) {
                    const int i = tid + q * nthr;
                    off2[q] = pending && i < G ? (red & 1) * G + i : -1;
                }
                if (!poll_tagged<kAresEdge, kAresPoll>(xbuf, off1, serial, x1, part64, off2, (uint32_t)red + 1u, x2,
                                                       a.sc))
                    gave_up = 1;
#pragma unroll
                for (int q = 0; q < kAresPoll; ++q) pv = off2[q] >= 0 && (uint32_t)x2[q] > pv ? (uint32_t)x2[q] : pv;
            }
            // ---- the pending check's decision (wmax was last read before this
            // chunk's sweeps, each of which ends at a block barrier)
            if (pending) {
                block_max_put(wmax, pv);
                __syncthreads();
                if (gave_up) return;
                R_bits = block_max_get(wmax);
                ++red;
                pending = false;
                const float rho = __uint_as_float(R_bits) / bA;
                const bool stop = !(rho >= a.tol);
                if (stop || kc >= a.max_sweeps) {
                    // JAC_ENAN : JAC_OK : JAC_ENOCONV; the result is u_kc, this chunk's input
                    status = stop ? ((rho != rho) ? -5 : 0) : -4;
                    cur = in;
                    k = kc;
                    break;
                }
            }
            // ---- the halos of the next chunk, in all three copies
#pragma unroll
            for (int p = 0; p < kAresEdge; ++p)
                if (roff[p] >= 0) {
                    const float v = __uint_as_float((uint32_t)x1[p]);
                    lds[rdst[p]] = v;
                    lds[RB + rdst[p]] = v;
                    lds[2 * RB + rdst[p]] = v;
                }
            __syncthreads();
            if (gave_up) return;
            // ---- a check point: the residual of u_k, whose halos are now the
            // neighbours' u_k; the block's partial goes out for the next exchange
            if (done == 0) {
                uint32_t m = 0;
#define JAC_ARES_CHECK(NQ) m = res_check<NQ>(lds, ob * 4, lp * 4, at, info, bv, r)
                JAC_RES_NQ(JAC_ARES_CHECK)
#undef JAC_ARES_CHECK
                block_max_put(wmax, m);
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(&part64[(int64_t)(red & 1) * G + blockIdx.x],
                                       ((uint64_t)(red + 1) << 32) | block_max_get(wmax), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                pending = true;
                kc = k;
            }
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
    // the field: each tile of the current iterate, into the buffer u^n came from
    for (int q = 0; q < ng; ++q) {
        const AresTile T = ares_tile(t0 + q, N, TX, TY, ntx);
        float* dst = (a.cur0 ? a.u1 : a.u0) + g.origin + (int64_t)T.y0 * P + T.x0;
        const int ob = cur * RB + q * R;
        for (int k = tid; k < T.w * T.h; k += nthr) {
            const int i = k / T.w, j = k - i * T.w;
            dst[(int64_t)i * P + j] = lds[ob + (1 + i) * lp + 1 + j];
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
                          uint64_t* xchg, int64_t xchg_words, void* out, int nsteps, int cur0, bool async_mode, int D,
                          int L, int tile_x, int tile_y, int side, int64_t max_sweeps, int cus, int* grid_used,
                          hipStream_t stream) {
    const int N = sa.g.N;
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
    a.xchg = xchg;
    a.out = reinterpret_cast<PersistOut*>(out);
    a.nsteps = nsteps;
    a.cur0 = cur0;
    a.async_mode = async_mode ? 1 : 0;
    a.D = D;
    a.L = L;
    a.sc = sa.sc;
    a.group = 1;
    a.max_sweeps = max_sweeps;
    int dev = 0, max_lds = 0;
    const bool have_lds = hipGetDevice(&dev) == hipSuccess &&
                          hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess;
    // Grids whose tiles all fit one round of co-resident blocks keep them
    // resident: k_persist_res for the exact kernels, k_persist_ares for the
    // block-asynchronous one; otherwise tiles are re-staged (k_persist).
    // Exact resident tiles are square, side T: the band_rows option, else the
    // smallest of 16, 32, 64 that fits (smaller tiles put more CUs on the
    // grid).  A tile is at least H = D + 1 cells on each side (a ragged last
    // tile too), the region's interior (T + 2H - 2)^2 fits the block's cells,
    // the region and the exchange maps its LDS, the exchange its words.
    bool resident = false;
    int rgrid = 0, T = 0;
    const int H = D + 1;
    size_t rlds = 0;
    if (!async_mode) {
        const int sides[3] = {16, 32, 64};
        for (int si = 0; si < 3 && !resident && have_lds; ++si) {
            T = side > 0 ? side : sides[si];
            const int64_t nt = (int64_t)((N + T - 1) / T) * ((N + T - 1) / T);
            const int R = (T + 2 * H) * (T + 2 * H);
            // two iterates, s, a dummy word, the publish and refill maps
            rlds = (size_t)(3 * R + 1 + 8 * H * T + 4 * H * H) * sizeof(float);
            int per_cu = 0;
            if (H <= T && (N % T == 0 || N % T >= H) && (T + 2 * H - 2) * (T + 2 * H - 2) <= kResThreads * kResCells &&
                4 * H * T <= kResThreads * kResPub && 4 * H * T + 4 * H * H <= kResThreads * kResRef &&
                rlds <= (size_t)max_lds &&
                (sa.fastdiv
                     ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_res<true>, kResThreads, rlds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_res<false>, kResThreads,
                                                                    rlds)) == hipSuccess &&
                per_cu > 0 && nt <= (int64_t)cus * per_cu && nt <= kMaxPersistBlocks &&
                resident_exchange_words((int)nt, H, T) <= xchg_words) {
                resident = true;
                rgrid = (int)nt;
            }
            if (side > 0) break;
        }
    }
    // Block-asynchronous resident tiles are the tile_x x tile_y tiles of the
    // launch kernel, in groups of G consecutive tiles per block: the smallest
    // G of 1, 2, 4, 8, 16 (more blocks on small grids) and, for it, the
    // largest block of 1024 ... 64 threads with at most 9 cells and 2 edge
    // words per thread whose grid fits one round; three copies per tile in LDS.
    bool ares = false;
    int athr = 0, agroup = 1;
    size_t alds = 0;
    if (async_mode && have_lds) {
        const int TX = tile_x, TY = tile_y, TC = TX * TY;
        const int64_t ntiles = (int64_t)((N + TX - 1) / TX) * ((N + TY - 1) / TY);
        for (int G = 1; G <= 16 && !ares; G *= 2) {
            if (G > 1 && ntiles < 2 * (int64_t)G) break;  // groups larger than the grid gain nothing
            const int64_t nb = (ntiles + G - 1) / G;
            const size_t lds_g = (size_t)3 * G * (TX + 2) * (TY + 2) * sizeof(float);
            if (lds_g > (size_t)max_lds) break;
            // block sizes: one thread per cell (a multiple of 64, at most 1024), then
            // the powers of two below it (whole wavefronts: the block maxima read lane 63)
            const int64_t want = (int64_t)G * (TC > TX + TY ? TC : TX + TY);
            const int first = want >= kResThreads ? kResThreads : (int)((want + 63) / 64 * 64);
            int cand[8], nc = 0;
            cand[nc++] = first;
            for (int t = kResThreads; t >= 64; t /= 2)
                if (t < first) cand[nc++] = t;
            for (int ci = 0; ci < nc && !ares; ++ci) {
                const int thr = cand[ci];
                if ((int64_t)G * TC > (int64_t)thr * kResCells || (int64_t)G * (TX + TY) > thr) break;
                int per_cu = 0;
                if ((sa.fastdiv ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_ares<true>, thr,
                                                                              lds_g)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_persist_ares<false>, thr,
                                                                              lds_g)) == hipSuccess &&
                    per_cu > 0 && nb <= (int64_t)cus * per_cu && nb <= kMaxPersistBlocks &&
                    nb <= (int64_t)kAresPoll * thr && ares_exchange_words((int)ntiles, TX, TY) <= xchg_words) {
                    ares = true;
                    athr = thr;
                    agroup = G;
                    alds = lds_g;
                    rgrid = (int)nb;
                }
            }
        }
    }
    PersistPlan p;
    if (resident) {
        a.tx = a.ty = T;
        a.lds_cells = 0;
        *grid_used = rgrid;
    } else if (ares) {
        a.tx = tile_x;
        a.ty = tile_y;
        a.group = agroup;
        a.lds_cells = 0;
        *grid_used = rgrid;
    } else {
        hipError_t e = persist_plan(N, D, async_mode, tile_x, tile_y, side, sa.fastdiv != 0, cus, &p);
        if (e != hipSuccess) return e;
        a.tx = p.tx;
        a.ty = p.ty;
        a.lds_cells = p.cells;
        *grid_used = p.grid;
    }
    // clear the barrier words (release, error) and the grid's flag lines with kernel fills
    hipError_t e = launch_fill(reinterpret_cast<float*>(&sa.sc->bar_release), 48, 0.0f, stream);
    if (e == hipSuccess)
        e = launch_fill(reinterpret_cast<float*>(scratch_flags(sa.sc)), (int64_t)(*grid_used) * kFlagStride, 0.0f,
                        stream);
    // tags of an earlier solve must not match: clear the exchange words and
    // the 2 x grid tagged partial words
    const int64_t xwords =
        resident ? resident_exchange_words(rgrid, H, T)
                 : ares ? ares_exchange_words((int)((int64_t)((N + tile_x - 1) / tile_x) * ((N + tile_y - 1) / tile_y)),
                                              tile_x, tile_y)
                        : 0;
    if (e == hipSuccess && xwords > 0) e = launch_fill(reinterpret_cast<float*>(xchg), 2 * xwords, 0.0f, stream);
    if (e == hipSuccess && (resident || ares))
        e = launch_fill(reinterpret_cast<float*>(partial), 4 * (int64_t)rgrid, 0.0f, stream);
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    if (resident) {
        const void* fr = sa.fastdiv ? reinterpret_cast<const void*>(k_persist_res<true>)
                                    : reinterpret_cast<const void*>(k_persist_res<false>);
        return hipLaunchCooperativeKernel(fr, dim3(rgrid), dim3(kResThreads), args, (unsigned)rlds, stream);
    }
    if (ares) {
        const void* fa = sa.fastdiv ? reinterpret_cast<const void*>(k_persist_ares<true>)
                                    : reinterpret_cast<const void*>(k_persist_ares<false>);
        return hipLaunchCooperativeKernel(fa, dim3(rgrid), dim3(athr), args, (unsigned)alds, stream);
    }
    const void* fn = sa.fastdiv ? reinterpret_cast<const void*>(k_persist<true>)
                                : reinterpret_cast<const void*>(k_persist<false>);
    return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kPersistThreads), args, (unsigned)p.lds, stream);
}

size_t persist_out_bytes() { return sizeof(PersistOut); }

}  // namespace jac
