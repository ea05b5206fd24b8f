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
    *grid_used = p.grid;
    // clear the barrier words (release, error) and the grid's flag lines with kernel fills
    e = launch_fill(reinterpret_cast<float*>(&sa.sc->bar_release), 48, 0.0f, stream);
    if (e == hipSuccess)
        e = launch_fill(reinterpret_cast<float*>(scratch_flags(sa.sc)), (int64_t)p.grid * kFlagStride, 0.0f, stream);
    if (e != hipSuccess) return e;
    void* args[] = {&a};
    const void* fn = sa.fastdiv ? reinterpret_cast<const void*>(k_persist<true>)
                                : reinterpret_cast<const void*>(k_persist<false>);
    return hipLaunchCooperativeKernel(fn, dim3(p.grid), dim3(kPersistThreads), args, (unsigned)p.lds, stream);
}

size_t persist_out_bytes() { return sizeof(PersistOut); }

}  // namespace jac
