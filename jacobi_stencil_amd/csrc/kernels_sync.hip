// kernels_sync.hip -- set-up kernels, the right-hand side, the synchronous
// sweep (kernel a) with the residual check fused into it, and the standalone
// residual.
//
// Synchronous sweep (page "stencil-jacobian.vercel.app", section 02, the
// synchronous strategy: every point of sweep k+1 reads only sweep k, two
// ping-pong buffers, one launch per sweep; fused right-hand side so a sweep
// moves 12 bytes per point: read u_k, read b, write u_{k+1}).
//
// MI355X mapping: a wavefront owns 256 consecutive columns (4 per lane, one
// 16-byte load per row) and walks down H rows keeping the rows above and below
// in registers, so each row of u is read from memory about once; the west and
// east neighbours of a lane's 4 columns are single-float loads that hit the
// cache lines its neighbours just fetched.  Four wavefronts of a block take four
// consecutive row bands of the same 256 columns.
#include "jacobi_internal.h"

namespace jac {

// ------------------------------------------------------------ set-up

__global__ void k_fill(float* __restrict__ p, int64_t n, float v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// Top ghost row (row -1, columns 0..N-1) = 100; the rest of the ring is the
// zero padding already written by k_fill.
__global__ void k_ghost_top(float* __restrict__ u, Geom g) {
    int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j < g.N) u[g.origin - g.P + j] = kTop;
}

hipError_t launch_ghosts(float* u, const Geom& g, hipStream_t s) {
    hipLaunchKernelGGL(k_ghost_top, dim3((g.N + 255) / 256), dim3(256), 0, s, u, g);
    return hipGetLastError();
}

// ------------------------------------------------------------ right-hand side

// b = u^n + s for every unknown, and per-block maxima of |b + r*g| (g = 100
// on row 0) for ||b_A||_inf.  One thread per 4 columns of one row; the grid
// is (column groups) x (rows).  KEEP_U (the unfused sweep): the plane gets a
// copy of u^n instead of b, the norm is the same.
template <bool KEEP_U>
__global__ __launch_bounds__(256) void k_rhs(const float* __restrict__ u, const float* __restrict__ src,
                                             float* __restrict__ b, StepArgs a) {
    const Geom g = a.g;
    const int col0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    uint32_t m = 0;
    for (int i = blockIdx.y; i < g.N; i += gridDim.y) {
        if (col0 >= g.N) break;
        const int64_t o = g.origin + (int64_t)i * g.P + col0;
        float4 uu = ld4_nt(u + o);
        float4 ss = ld4_nt(src + o);
        float4 bb;
        bb.x = uu.x + ss.x;
        bb.y = uu.y + ss.y;
        bb.z = uu.z + ss.z;
        bb.w = uu.w + ss.w;
        const float rg = a.r * (i == 0 ? kTop : 0.0f);
        const float vb[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (col0 + c < g.N) {
                uint32_t v = __float_as_uint(fabsf(vb[c] + rg));
                m = m > v ? m : v;
            }
        }
        const float4 out = KEEP_U ? uu : bb;
        if (col0 + 4 <= g.N) {
            st4_nt(b + o, out);
        } else {
            const float vo[4] = {out.x, out.y, out.z, out.w};
            for (int c = 0; c < 4; ++c)
                if (col0 + c < g.N) b[o + c] = vo[c];
        }
    }
    store_block_max<4>(m, a.sc, (int64_t)blockIdx.y * gridDim.x + blockIdx.x);
}

int64_t rhs_blocks(int N) {
    const int64_t gx = (N + 1023) / 1024;
    const int64_t gy = N < 1024 ? N : 1024;
    return gx * gy;
}

hipError_t launch_rhs(const float* u, const float* src, float* b, bool keep_u, const StepArgs& a, hipStream_t s) {
    const int gx = (a.g.N + 1023) / 1024;
    int gy = a.g.N < 1024 ? a.g.N : 1024;
    if (keep_u)
        hipLaunchKernelGGL(k_rhs<true>, dim3(gx, gy), dim3(256), 0, s, u, src, b, a);
    else
        hipLaunchKernelGGL(k_rhs<false>, dim3(gx, gy), dim3(256), 0, s, u, src, b, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ reductions

constexpr int kReduceThreads = 1024;

__device__ __forceinline__ uint32_t block_reduce_partials(const uint32_t* part, int64_t npart) {
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < npart; i += kReduceThreads) {
        const uint32_t v = part[i];
        m = m > v ? m : v;
    }
    m = wave_max_u32(m);
    __shared__ uint32_t w[kReduceThreads / 64];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t bm = w[0];
    for (int k = 1; k < kReduceThreads / 64; ++k) bm = bm > w[k] ? bm : w[k];
    __syncthreads();  // w is free again
    return bm;
}

__global__ __launch_bounds__(kReduceThreads) void k_reduce(int64_t npart, int norm, StepArgs a) {
    Scratch* sc = a.sc;
    if (!norm && sc->stop) return;  // the step stopped at an earlier check
    const uint32_t* part = scratch_partials(sc) + a.part_off;
    const uint32_t bm = block_reduce_partials(part, npart);
    // a second check of the same launch: the next npart slots
    const uint32_t bm2 = (!norm && a.slot2 >= 0) ? block_reduce_partials(part + npart, npart) : 0u;
    if (threadIdx.x == 0) {
        if (norm) {
            sc->bA_bits = bm;
            sc->stop = 0u;
            sc->check_seq = 0u;
            __hip_atomic_store(&a.mail->bA_bits, bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        } else {
            const float bA = __uint_as_float(sc->bA_bits);
            const float rho = __uint_as_float(bm) / bA;
            bool stop = !(rho >= a.tol);
            const uint32_t seq = sc->check_seq;
            const int slot = a.slot >= 0 ? a.slot : (int)(seq % (uint32_t)kRing);
            sc->check_seq = seq + 1u;
            __hip_atomic_store(&a.mail->R[slot], bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            if (a.slot2 >= 0) {
                // the host reads the first check before the second; either one stops the step
                const float rho2 = __uint_as_float(bm2) / bA;
                stop = stop || !(rho2 >= a.tol);
                sc->check_seq = seq + 2u;
                __hip_atomic_store(&a.mail->R[a.slot2], bm2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            }
            sc->stop = stop ? 1u : 0u;
        }
    }
}

hipError_t launch_reduce(int64_t npart, bool norm, const StepArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(kReduceThreads), 0, s, npart, norm ? 1 : 0, a);
    return hipGetLastError();
}

// ------------------------------------------------------------ sync sweep

constexpr int kSyncWaves = 4;

struct SyncTiles {
    int rows, tiles_x, tiles_y, blocks;
};

static SyncTiles sync_tiles(int N, int rows) {
    SyncTiles t;
    t.rows = rows;
    t.tiles_x = (N + 255) / 256;
    t.tiles_y = (N + kSyncWaves * t.rows - 1) / (kSyncWaves * t.rows);
    t.blocks = (t.tiles_x * t.tiles_y + 7) / 8 * 8;
    return t;
}

// One row of 4 columns: the sweep and/or the residual of the middle row.
template <bool DO_SWEEP, bool DO_CHECK, bool FAST>
__device__ __forceinline__ void sync_row(const float4& up, const float4& mid, const float4& dn, const float4& bb,
                                         float wl, float er, float r, float d, float y, float4& o4, uint32_t& m,
                                         int valid /* columns of the 4 that are unknowns */) {
    if (DO_CHECK) {
        uint32_t v0 = residual_bits(mid.x, mid.y, wl, up.x, dn.x, bb.x, r);
        uint32_t v1 = residual_bits(mid.y, mid.z, mid.x, up.y, dn.y, bb.y, r);
        uint32_t v2 = residual_bits(mid.z, mid.w, mid.y, up.z, dn.z, bb.z, r);
        uint32_t v3 = residual_bits(mid.w, er, mid.z, up.w, dn.w, bb.w, r);
        if (valid < 4) {
            if (valid < 2) v1 = 0;
            if (valid < 3) v2 = 0;
            v3 = 0;
        }
        uint32_t v01 = v0 > v1 ? v0 : v1, v23 = v2 > v3 ? v2 : v3;
        uint32_t v = v01 > v23 ? v01 : v23;
        m = m > v ? m : v;
    }
    if (DO_SWEEP) {
        o4.x = jacobi_update<FAST>(mid.y, wl, up.x, dn.x, bb.x, r, d, y);
        o4.y = jacobi_update<FAST>(mid.z, mid.x, up.y, dn.y, bb.y, r, d, y);
        o4.z = jacobi_update<FAST>(mid.w, mid.y, up.z, dn.z, bb.z, r, d, y);
        o4.w = jacobi_update<FAST>(er, mid.z, up.w, dn.w, bb.w, r, d, y);
    }
}

// The right-hand side of 4 columns: b itself, or (UNF, the unfused sweep)
// u^n + s formed on the fly, with the same single addition as the RHS kernel.
template <bool UNF, bool NT>
__device__ __forceinline__ float4 rhs4(const float* pb, const float* ps) {
    const float4 v = NT ? ld4_nt(pb) : ld4(pb);
    if (!UNF) return v;
    const float4 w = NT ? ld4_nt(ps) : ld4(ps);
    return make_float4(v.x + w.x, v.y + w.y, v.z + w.z, v.w + w.w);
}

// One sweep u_{k+1} = J(u_k).  With CHECK the same pass also measures the
// residual of u_k (the iterate it reads), which costs no extra memory traffic;
// RESID_ONLY measures the residual and writes nothing.  UNF: `bin` holds u^n
// and `sin` the source s, and b = u^n + s is formed per point -- the unfused
// baseline of page "stencil-jacobian.vercel.app", section 02 (16 bytes per
// point per sweep instead of 12); the results are identical.
template <bool CHECK, bool RESID_ONLY, bool FAST, bool UNF, int H>
__global__ __launch_bounds__(256) void k_sync(const float* __restrict__ uin, const float* __restrict__ bin,
                                              const float* __restrict__ sin, float* __restrict__ uout, StepArgs a) {
    constexpr bool SWEEP = !RESID_ONLY;
    constexpr bool CHK = CHECK || RESID_ONLY;
    if (a.sc->stop) return;  // a previous check already stopped the step
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tiles_x = (N + 255) / 256;
    const int tiles_y = (N + kSyncWaves * H - 1) / (kSyncWaves * H);
    const int t = xcd_logical_block(blockIdx.x, gridDim.x);
    const int wcol = (t % tiles_x) * 256;
    const int col0 = wcol + lane * 4;
    const int row0 = (t / tiles_x) * (kSyncWaves * H) + wave * H;
    const float r = a.r, d = a.d, y = a.y;
    uint32_t m = 0;
    if (t < tiles_x * tiles_y && row0 < N) {
        const int64_t o = g.origin + (int64_t)row0 * P + col0;
        const float* pu = uin + o;
        const float* pb = bin + o;
        const float* ps = UNF ? sin + o : nullptr;
        float* po = uout + o;
        if (wcol + 256 <= N && row0 + H <= N) {
            // interior wavefront: 256 full columns, H full rows.  West/east
            // neighbours come from the adjacent lanes (DPP); lanes 0 and 63 take
            // the columns just outside the wavefront, loaded for all H rows up
            // front (lane i holds row i).  Rows and b stream with nontemporal
            // loads, except the two rows shared with the bands above and below.
            const int erow = lane < H ? lane : 0;
            const float wedge = uin[g.origin + (int64_t)(row0 + erow) * P + wcol - 1];
            const float eedge = uin[g.origin + (int64_t)(row0 + erow) * P + wcol + 256];
            float4 up = ld4(pu - P);
            float4 mid = ld4_nt(pu);
            // rows in groups of G (up to 8): the loads of a group are all in
            // flight before its first row is computed
            constexpr int G = H < 8 ? H : 8;
#pragma unroll
            for (int i0 = 0; i0 < H; i0 += G) {
                float4 dn[G], bb[G];
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const int i = i0 + k;
                    dn[k] = (i == H - 1) ? ld4(pu + (int64_t)(i + 1) * P) : ld4_nt(pu + (int64_t)(i + 1) * P);
                    bb[k] = rhs4<UNF, true>(pb + (int64_t)i * P, UNF ? ps + (int64_t)i * P : nullptr);
                }
#pragma unroll
                for (int k = 0; k < G; ++k) {
                    const int i = i0 + k;
                    float wl = from_left(mid.w);
                    float er = from_right(mid.x);
                    const float ws = __shfl(wedge, i, 64);
                    const float es = __shfl(eedge, i, 64);
                    wl = lane == 0 ? ws : wl;
                    er = lane == 63 ? es : er;
                    float4 o4;
                    sync_row<SWEEP, CHK, FAST>(up, mid, dn[k], bb[k], wl, er, r, d, y, o4, m, 4);
                    if (SWEEP) st4_nt(po + (int64_t)i * P, o4);
                    up = mid;
                    mid = dn[k];
                }
            }
        } else if (col0 < N) {
            // edge wavefront: ragged rows and/or columns
            const int rows = (N - row0) < H ? (N - row0) : H;
            const int valid = (N - col0) < 4 ? (N - col0) : 4;
            float4 up = ld4(pu - P);
            float4 mid = ld4(pu);
            for (int i = 0; i < rows; ++i) {
                const float4 dn = ld4(pu + (int64_t)(i + 1) * P);
                const float4 bb = rhs4<UNF, false>(pb + (int64_t)i * P, UNF ? ps + (int64_t)i * P : nullptr);
                const float wl = pu[(int64_t)i * P - 1];
                const float er = pu[(int64_t)i * P + 4];
                float4 o4;
                sync_row<SWEEP, CHK, FAST>(up, mid, dn, bb, wl, er, r, d, y, o4, m, valid);
                if (SWEEP) {
                    float* q = po + (int64_t)i * P;
                    if (valid == 4) {
                        *reinterpret_cast<float4*>(q) = o4;
                    } else {
                        q[0] = o4.x;
                        if (valid > 1) q[1] = o4.y;
                        if (valid > 2) q[2] = o4.z;
                    }
                }
                up = mid;
                mid = dn;
            }
        }
    }
    if (CHK) store_block_max<kSyncWaves>(m, a.sc, blockIdx.x);
}

int64_t sync_blocks(int N, int rows) { return sync_tiles(N, rows).blocks; }

// Rows per wavefront.  16 by default (each row of u read about once, the two
// rows shared with the neighbouring bands excepted), or 4 on grids too small to
// give the GPU a thousand 16-row wavefronts -- there a sweep is bound by the
// latency of a wavefront's row stream, not by bandwidth.  64 when those longer
// bands make one balanced round: the same number of workgroups on every CU, at
// least four (one wavefront per SIMD each) and no more than fit at once.  Then
// fewer shared rows are re-read and more loads are in flight per wavefront
// (N = 8192: 140 us per sweep against 148 at 16 rows); otherwise the longer
// bands lose to their uneven last round (N = 6144 to 16384: 2-13 % slower).
// At most 64: a wavefront preloads its two edge columns one row per lane.
int sync_rows_for(int N, int cus) {
    const int64_t strips = (N + 255) / 256;
    const int64_t blocks64 = sync_blocks(N, 64);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_sync<true, false, true, false, 64>, 64 * kSyncWaves,
                                                     0) != hipSuccess)
        per_cu = 0;
    if (cus > 0 && blocks64 % cus == 0 && blocks64 / cus >= 4 && blocks64 / cus <= per_cu) return 64;
    if (strips * ((N + 15) / 16) >= 1024) return 16;
    return 4;
}

template <bool UNF, int H>
static void launch_sync_t(const float* uin, const float* b, const float* src, float* uout, bool check,
                          const StepArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if (check) {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_sync<true, false, true, UNF, H>), grid, block, 0, s, uin, b, src, uout, a);
        else
            hipLaunchKernelGGL((k_sync<true, false, false, UNF, H>), grid, block, 0, s, uin, b, src, uout, a);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_sync<false, false, true, UNF, H>), grid, block, 0, s, uin, b, src, uout, a);
        else
            hipLaunchKernelGGL((k_sync<false, false, false, UNF, H>), grid, block, 0, s, uin, b, src, uout, a);
    }
}

hipError_t launch_sync(const float* uin, const float* b, const float* src, float* uout, bool check, int rows,
                       const StepArgs& a, hipStream_t s) {
    SyncTiles t = sync_tiles(a.g.N, rows);
    const dim3 grid(t.blocks), block(64 * kSyncWaves);
    if (t.rows == 64) {
        if (src)
            launch_sync_t<true, 64>(uin, b, src, uout, check, a, grid, block, s);
        else
            launch_sync_t<false, 64>(uin, b, nullptr, uout, check, a, grid, block, s);
    } else if (t.rows == 16) {
        if (src)
            launch_sync_t<true, 16>(uin, b, src, uout, check, a, grid, block, s);
        else
            launch_sync_t<false, 16>(uin, b, nullptr, uout, check, a, grid, block, s);
    } else {
        if (src)
            launch_sync_t<true, 4>(uin, b, src, uout, check, a, grid, block, s);
        else
            launch_sync_t<false, 4>(uin, b, nullptr, uout, check, a, grid, block, s);
    }
    return hipGetLastError();
}

template <int H>
static void launch_residual_t(const float* u, const float* b, const float* src, const StepArgs& a, dim3 grid,
                              hipStream_t s) {
    const dim3 block(64 * kSyncWaves);
    if (src)
        hipLaunchKernelGGL((k_sync<false, true, false, true, H>), grid, block, 0, s, u, b, src, (float*)nullptr, a);
    else
        hipLaunchKernelGGL((k_sync<false, true, false, false, H>), grid, block, 0, s, u, b, (const float*)nullptr,
                           (float*)nullptr, a);
}

hipError_t launch_residual(const float* u, const float* b, const float* src, int rows, const StepArgs& a,
                           hipStream_t s) {
    SyncTiles t = sync_tiles(a.g.N, rows);
    if (t.rows == 64)
        launch_residual_t<64>(u, b, src, a, dim3(t.blocks), s);
    else if (t.rows == 16)
        launch_residual_t<16>(u, b, src, a, dim3(t.blocks), s);
    else
        launch_residual_t<4>(u, b, src, a, dim3(t.blocks), s);
    return hipGetLastError();
}

// ------------------------------------------------------------ division check

__global__ __launch_bounds__(256) void k_verify_div(float d, float y, Scratch* sc) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t bad = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
        const uint32_t bits = (uint32_t)i;
        // the numerators the host keeps away from the fast quotient: Inf, NaN, -0
        if ((bits & 0x7F800000u) == 0x7F800000u || bits == 0x80000000u) continue;
        const float n = __uint_as_float(bits);
        const float q = div_d<false>(n, d, y);
        const float f = div_d<true>(n, d, y);
        bad += __float_as_uint(q) == __float_as_uint(f) ? 0u : 1u;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bad += (uint32_t)__shfl_xor((int)bad, o, 64);
    if ((threadIdx.x & 63) == 0 && bad) atomicAdd(&sc->div_bad, bad);  // only where it failed
}

hipError_t launch_verify_div(float d, float y, Scratch* sc, hipStream_t s) {
    hipLaunchKernelGGL(k_verify_div, dim3(8192), dim3(256), 0, s, d, y, sc);
    return hipGetLastError();
}

}  // namespace jac
