// kernels_async.hip -- block-asynchronous relaxation (kernel c).
//
// The method (page "stencil-jacobian.vercel.app", section 01 "block-
// asynchronous" and section 02, after Anzt et al.; also Islam & Wang,
// "Hierarchical Jacobi Iteration for Structured Matrices on GPUs using Shared
// Memory", section 3): each block loads its tile plus a one-cell halo into
// on-chip memory and performs D Jacobi sweeps on the tile with the halo
// frozen, then writes the tile back.  Values read across a tile edge are up to
// D-1 sweeps old; with D = 1 this is the synchronous sweep.
//
// Overlapping subdomains (Islam & Wang, sections 3.5 and 4): with overlap o a
// tile iterates on itself widened by o cells per side (clipped to the grid),
// the frozen ring lying one cell outside that, and writes back only its own
// points; points near a tile edge then see fresher neighbours.  o = 0 is the
// plain block-async launch; o >= D - 1 reproduces D synchronous sweeps.
//
// Three forms, chosen by tile shape (results identical): four columns per lane
// in 256-column strips (widths dividing 256, heights 4 and 8), one column per
// lane in 64-column strips (widths dividing 64, heights up to 32), and the LDS
// form below for every other shape and for overlap.
//
// LDS form: tiles of tile_x columns by tile_y rows start at unknown (0, 0), the
// last ones in each direction clipped to the grid.  The halo comes from the
// iterate the launch reads (u_k, ping-pong between launches), so a launch is a
// deterministic function of u_k and the result does not depend on scheduling.
// One workgroup of 256 threads per tile; the tile and its halo live twice in
// LDS (in-tile ping-pong; the halo is copied into both and never written);
// each thread keeps b for its points in registers; a barrier separates the
// in-tile sweeps.  Every point update uses the same float32 operations, in the
// same order, as the synchronous sweep.
#include "jacobi_internal.h"

namespace jac {

constexpr int kAsyncThreads = 256;
constexpr int kAsyncMaxPts = 4096;                          // tile_x * tile_y
constexpr int kAsyncPerThread = kAsyncMaxPts / kAsyncThreads;  // points per thread, at most

template <bool CHK, bool FAST>
__global__ __launch_bounds__(kAsyncThreads) void k_async(const float* __restrict__ uin,
                                                         const float* __restrict__ bin,
                                                         float* __restrict__ uout, StepArgs a, int tx,
                                                         int ty, int D, int o) {
    extern __shared__ float lds[];
    if (a.sc->stop) return;  // a previous check already stopped the step
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int ntx = (N + tx - 1) / tx, nty = (N + ty - 1) / ty;
    const int t = xcd_logical_block(blockIdx.x, gridDim.x);
    uint32_t m = 0;
    if (t < ntx * nty) {
        const int x0 = (t % ntx) * tx, y0 = (t / ntx) * ty;
        const int x1 = (x0 + tx <= N) ? x0 + tx : N;  // owned columns [x0, x1), rows [y0, y1)
        const int y1 = (y0 + ty <= N) ? y0 + ty : N;
        const int ex0 = x0 - o < 0 ? 0 : x0 - o;      // the region worked on
        const int ex1 = x1 + o > N ? N : x1 + o;
        const int ey0 = y0 - o < 0 ? 0 : y0 - o;
        const int ey1 = y1 + o > N ? N : y1 + o;
        const int w = ex1 - ex0, h = ey1 - ey0;
        const int lp = w + 2;                         // LDS row pitch: region plus halo
        const int ln = lp * (h + 2);
        float* A = lds;
        float* B = lds + ln;
        const float r = a.r, d = a.d, y = a.y;
        // region and halo: LDS (a, c) is unknown (ey0 + a - 1, ex0 + c - 1);
        // the halo ring is neighbouring tiles' u_k or the ghost ring
        const float* src = uin + g.origin + (int64_t)(ey0 - 1) * P + (ex0 - 1);
        for (int k = threadIdx.x; k < ln; k += kAsyncThreads) {
            const int ra = k / lp, ca = k - ra * lp;
            const float v = src[(int64_t)ra * P + ca];
            A[k] = v;
            B[k] = v;
        }
        const int npts = w * h;
        // this thread's points, once: LDS offset, and (region row << 16 | column)
        // with bit 31 set for a point the tile owns; the sweep loop then does no
        // index arithmetic
        const int nq = (npts + kAsyncThreads - 1) / kAsyncThreads;  // uniform
        float bb[kAsyncPerThread];
        int cl[kAsyncPerThread];
        uint32_t ij[kAsyncPerThread];
#pragma unroll
        for (int q = 0; q < kAsyncPerThread; ++q) {
            const int p = threadIdx.x + q * kAsyncThreads;
            bb[q] = 0.0f;
            cl[q] = lp + 1;
            ij[q] = 0u;
            if (p < npts) {
                const int i = p / w, j = p - (p / w) * w;
                cl[q] = (i + 1) * lp + (j + 1);
                const bool own = ey0 + i >= y0 && ey0 + i < y1 && ex0 + j >= x0 && ex0 + j < x1;
                ij[q] = ((uint32_t)i << 16) | (uint32_t)j | (own ? 0x80000000u : 0u);
                bb[q] = bin[g.origin + (int64_t)(ey0 + i) * P + (ex0 + j)];
            }
        }
        __syncthreads();
        if (CHK) {
            // residual of u_k on the tile's own points (the halo is u_k too)
#pragma unroll
            for (int q = 0; q < kAsyncPerThread; ++q) {
                if (q < nq && (ij[q] & 0x80000000u)) {
                    const int c = cl[q];
                    const uint32_t v = residual_bits(A[c], A[c + 1], A[c - 1], A[c - lp], A[c + lp], bb[q], r);
                    m = m > v ? m : v;
                }
            }
        }
        float* cur = A;
        float* nxt = B;
        for (int s = 0; s < D; ++s) {
#pragma unroll
            for (int q = 0; q < kAsyncPerThread; ++q) {
                if (q < nq && (int)threadIdx.x + q * kAsyncThreads < npts) {
                    const int c = cl[q];
                    nxt[c] = jacobi_update<FAST>(cur[c + 1], cur[c - 1], cur[c - lp], cur[c + lp], bb[q], r, d, y);
                }
            }
            __syncthreads();
            float* tmp = cur;
            cur = nxt;
            nxt = tmp;
        }
        float* dst = uout + g.origin + (int64_t)ey0 * P + ex0;
#pragma unroll
        for (int q = 0; q < kAsyncPerThread; ++q) {
            if (q < nq && (ij[q] & 0x80000000u)) {
                const int i = (int)((ij[q] >> 16) & 0x7FFFu), j = (int)(ij[q] & 0xFFFFu);
                dst[(int64_t)i * P + j] = cur[cl[q]];
            }
        }
    }
    if (CHK) store_block_max<kAsyncThreads / 64>(m, a.sc, blockIdx.x);
}

// ---- register form: tile widths dividing 64, heights 4, 8, 16 or 32, no overlap
//
// One wavefront owns a strip of 64 columns x TY rows, one column per lane, and
// keeps the strip's TY values of u, of b and of the frozen halo in registers;
// the strip holds 64 / tile_x whole tiles side by side.  North and south
// neighbours are the lane's own rows (rows Y-1 and Y+TY are the frozen halo
// rows, read once); west and east neighbours come from the adjacent lanes by
// DPP shifts, except on a tile's edge columns, which read the frozen halo
// column instead: the neighbouring tile's (or neighbouring strip's) u_k,
// captured before the first sweep.  A sweep updates the rows in place from the
// top, keeping the old value of the row above.  Lanes past column N-1 and rows
// past N-1 hold the zero ghost column / row and padding and are never updated,
// which also gives clipped tiles their ghost halo.  No LDS, no barriers.
constexpr int kWaveStrip = 64;

bool async_wave_form(int tx, int ty, int o) {
    return o == 0 && (tx == 8 || tx == 16 || tx == 32 || tx == 64) && (ty == 4 || ty == 8 || ty == 16 || ty == 32);
}

template <int TY, bool EDGE, bool CHK, bool FAST, bool SMP>
__device__ __forceinline__ uint32_t async_strip(const float* __restrict__ uin, const float* __restrict__ bin,
                                                float* __restrict__ uout, const StepArgs& a, int tx, int D, int X,
                                                int Y) {
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int lane = threadIdx.x & 63;
    const int col = X + lane;
    const bool in_col = !EDGE || col < N;
    const bool west = (lane & (tx - 1)) == 0, east = (lane & (tx - 1)) == tx - 1;
    const float r = a.r, d = a.d, y = a.y;
    const float* pu = uin + g.origin + (int64_t)Y * P + col;
    const float* pb = bin + g.origin + (int64_t)Y * P + col;
    float cur[TY], bb[TY], hx[TY];
    const float top = pu[-(int64_t)P];
    const float bot = pu[(int64_t)TY * P];
#pragma unroll
    for (int i = 0; i < TY; ++i) {
        cur[i] = pu[(int64_t)i * P];
        bb[i] = pb[(int64_t)i * P];
    }
    // the columns just outside the strip, lane i holding row i
    const int er = lane < TY ? lane : 0;
    const float wcol = uin[g.origin + (int64_t)(Y + er) * P + X - 1];
    const float ecol = uin[g.origin + (int64_t)(Y + er) * P + X + kWaveStrip];
#pragma unroll
    for (int i = 0; i < TY; ++i) {
        const float l = from_left(cur[i]), rr = from_right(cur[i]);
        const float ws = __shfl(wcol, i, 64), es = __shfl(ecol, i, 64);
        hx[i] = west ? (lane == 0 ? ws : l) : (east ? (lane == 63 ? es : rr) : 0.0f);
    }
    uint32_t m = 0;
    // One sweep from `src` into `dst` (rows past the grid and lanes past
    // column N-1 keep their values); with `check` the residual of u_k is taken
    // from the same stencil on the way.  Two sweeps per trip with the roles
    // swapped, so no register is copied back between sweeps.
    auto sweep = [&](const float (&src)[TY], float (&dst)[TY], bool check) {
#pragma unroll
        for (int i = 0; i < TY; ++i) {
            const float c = src[i];
            const float l = from_left(c), rr = from_right(c);
            const float W = west ? hx[i] : l;
            const float E = east ? hx[i] : rr;
            const float Nn = i > 0 ? src[i - 1] : top;
            const float Sn = i + 1 < TY ? src[i + 1] : bot;
            const bool live = (!EDGE || Y + i < N) && in_col;
            if (CHK && check && (!SMP || (i & 7) == 0)) {  // SMP: every 8th row (the strip starts on one)
                const uint32_t e = residual_bits(c, E, W, Nn, Sn, bb[i], r);
                if (live) m = m > e ? m : e;
            }
            const float v = jacobi_update<FAST>(E, W, Nn, Sn, bb[i], r, d, y);
            dst[i] = live ? v : c;
        }
    };
    float alt[TY];
    int s = 0;
    for (; s + 2 <= D; s += 2) {
        sweep(cur, alt, s == 0);
        sweep(alt, cur, false);
    }
    if (s < D) {
        sweep(cur, alt, s == 0);
#pragma unroll
        for (int i = 0; i < TY; ++i) cur[i] = alt[i];
    }
    float* po = uout + g.origin + (int64_t)Y * P + col;
#pragma unroll
    for (int i = 0; i < TY; ++i)
        if ((!EDGE || Y + i < N) && in_col) po[(int64_t)i * P] = cur[i];
    return m;
}

template <int TY, bool CHK, bool FAST, bool SMP = false>
__global__ __launch_bounds__(256) void k_async_wave(const float* __restrict__ uin, const float* __restrict__ bin,
                                                    float* __restrict__ uout, StepArgs a, int tx, int D) {
    if (a.sc->stop) return;  // a previous check already stopped the step
    const int N = a.g.N;
    const int sx = (N + kWaveStrip - 1) / kWaveStrip, sy = (N + TY - 1) / TY;
    const int wid = xcd_logical_block(blockIdx.x, gridDim.x) * 4 + (int)(threadIdx.x >> 6);
    uint32_t m = 0;
    if (wid < sx * sy) {
        const int X = (wid % sx) * kWaveStrip, Y = (wid / sx) * TY;
        if (X + kWaveStrip <= N && Y + TY <= N)
            m = async_strip<TY, false, CHK, FAST, SMP>(uin, bin, uout, a, tx, D, X, Y);
        else
            m = async_strip<TY, true, CHK, FAST, SMP>(uin, bin, uout, a, tx, D, X, Y);
    }
    if (CHK) store_block_max<4>(m, a.sc, blockIdx.x);
}

// ---- four-column register form: tile widths 4..256 dividing 256, heights 4 and 8, no overlap
//
// As above, but each lane holds 4 adjacent columns (one 16-byte load per row)
// and a wavefront owns a strip of 256 columns.  The west and east neighbours of
// a lane's inner columns are in its own registers; only column 0 of the lane
// takes a DPP shift from the lane to its left and column 3 one from the lane to
// its right, and since tile widths are multiples of 4, a tile edge can only fall
// on those two columns -- so the frozen halo is kept, and selected, for them
// alone.  Per point-sweep: the 8 instructions of the update plus half a shift
// and half a select, against 2 and 2 in the one-column form.
constexpr int kWideStrip = 256;

// A four-column grid has a quarter of the one-column form's wavefronts; it is
// used only where that still leaves two per SIMD (MI355X has 1024): on smaller
// grids the idle SIMDs cost more than the instructions it saves (N = 1024,
// D4 at 32 x 8 tiles: 7.2 ms per ten steps against 6.4 in the one-column form;
// N = 2048: 10.3 against 12.4).
constexpr int64_t kWideMinWaves = 2048;

bool async_wide_form(int N, int tx, int ty, int o) {
    if (!(o == 0 && tx % 4 == 0 && kWideStrip % tx == 0 && (ty == 4 || ty == 8))) return false;
    const int64_t waves = (int64_t)((N + kWideStrip - 1) / kWideStrip) * ((N + ty - 1) / ty);
    return waves >= kWideMinWaves;
}

// Checking launches of D sweeps on this tiling take a check's residual on
// every 8th row when asked (row mask 7, constant-divisor path): the one-lane
// strip kernel with strips a multiple of 8 rows tall, for D <= 8 (deeper
// launches of that variant ran slower than the residual they save).
bool async_samples_rows(int N, int tx, int ty, int o, int D) {
    return !async_wide_form(N, tx, ty, o) && async_wave_form(tx, ty, o) && ty % 8 == 0 && D <= 8;
}

template <int TY, bool EDGE, bool CHK, bool FAST>
__device__ __forceinline__ uint32_t async_wide_strip(const float* __restrict__ uin, const float* __restrict__ bin,
                                                     float* __restrict__ uout, const StepArgs& a, int tx, int D,
                                                     int X, int Y) {
    const Geom g = a.g;
    const int N = g.N, P = g.P;
    const int lane = threadIdx.x & 63;
    const int c0 = X + 4 * lane;
    // columns of this lane that are unknowns (EDGE strips only reach past N)
    const bool in0 = !EDGE || c0 < N, in1 = !EDGE || c0 + 1 < N, in2 = !EDGE || c0 + 2 < N,
               in3 = !EDGE || c0 + 3 < N;
    const bool west = (c0 % tx) == 0, east = ((c0 + 4) % tx) == 0;
    const float r = a.r, d = a.d, y = a.y;
    const float* pu = uin + g.origin + (int64_t)Y * P + c0;
    const float* pb = bin + g.origin + (int64_t)Y * P + c0;
    float4 cur[TY], alt[TY], bb[TY];
    float hw[TY], he[TY];  // frozen halo of column 0 (west) and column 3 (east) on tile edges
    const float4 top = ld4(pu - P);
    const float4 bot = ld4(pu + (int64_t)TY * P);
#pragma unroll
    for (int i = 0; i < TY; ++i) {
        cur[i] = ld4(pu + (int64_t)i * P);
        bb[i] = ld4(pb + (int64_t)i * P);
    }
    // the columns just outside the strip, lane i holding row i
    const int er = lane < TY ? lane : 0;
    const float wcol = uin[g.origin + (int64_t)(Y + er) * P + X - 1];
    const float ecol = uin[g.origin + (int64_t)(Y + er) * P + X + kWideStrip];
#pragma unroll
    for (int i = 0; i < TY; ++i) {
        const float l = from_left(cur[i].w), rr = from_right(cur[i].x);
        const float ws = __shfl(wcol, i, 64), es = __shfl(ecol, i, 64);
        hw[i] = lane == 0 ? ws : l;
        he[i] = lane == 63 ? es : rr;
    }
    uint32_t m = 0;
    // Residual of u_k on row i, from the stencil the first sweep reads anyway.
    auto residual_row = [&](int i, const float4& c, const float4& n, const float4& sth, float W, float E) {
        uint32_t v0 = residual_bits(c.x, c.y, W, n.x, sth.x, bb[i].x, r);
        uint32_t v1 = residual_bits(c.y, c.z, c.x, n.y, sth.y, bb[i].y, r);
        uint32_t v2 = residual_bits(c.z, c.w, c.y, n.z, sth.z, bb[i].z, r);
        uint32_t v3 = residual_bits(c.w, E, c.z, n.w, sth.w, bb[i].w, r);
        if (EDGE) {
            const bool row = Y + i < N;
            v0 = (row && in0) ? v0 : 0u;
            v1 = (row && in1) ? v1 : 0u;
            v2 = (row && in2) ? v2 : 0u;
            v3 = (row && in3) ? v3 : 0u;
        }
        const uint32_t va = v0 > v1 ? v0 : v1, vb = v2 > v3 ? v2 : v3;
        const uint32_t v = va > vb ? va : vb;
        m = m > v ? m : v;
    };
    // One row i of a sweep: the new values from the old rows n (above), c
    // and sth (below); rows past the grid and columns past N-1 keep theirs.
    // With `check` the row's residual of u_k is taken on the way.
    auto update_row = [&](int i, const float4& c, const float4& n, const float4& sth, bool check) {
        const float l = from_left(c.w), rr = from_right(c.x);  // in every lane, then select
        const float W = west ? hw[i] : l;
        const float E = east ? he[i] : rr;
        if (CHK && check) residual_row(i, c, n, sth, W, E);
        float4 v;
        v.x = jacobi_update<FAST>(c.y, W, n.x, sth.x, bb[i].x, r, d, y);
        v.y = jacobi_update<FAST>(c.z, c.x, n.y, sth.y, bb[i].y, r, d, y);
        v.z = jacobi_update<FAST>(c.w, c.y, n.z, sth.z, bb[i].z, r, d, y);
        v.w = jacobi_update<FAST>(E, c.z, n.w, sth.w, bb[i].w, r, d, y);
        if (EDGE) {
            const bool row = Y + i < N;
            v.x = (row && in0) ? v.x : c.x;
            v.y = (row && in1) ? v.y : c.y;
            v.z = (row && in2) ? v.z : c.z;
            v.w = (row && in3) ? v.w : c.w;
        }
        return v;
    };
    // two sweeps per trip with the register sets swapped
    auto sweep = [&](const float4 (&src)[TY], float4 (&dst)[TY], bool check) {
#pragma unroll
        for (int i = 0; i < TY; ++i)
            dst[i] = update_row(i, src[i], i > 0 ? src[i - 1] : top, i + 1 < TY ? src[i + 1] : bot, check);
    };
    int s = 0;
    for (; s + 2 <= D; s += 2) {
        sweep(cur, alt, s == 0);
        sweep(alt, cur, false);
    }
    if (s < D) {
        sweep(cur, alt, s == 0);
#pragma unroll
        for (int i = 0; i < TY; ++i) cur[i] = alt[i];
    }
    float* po = uout + g.origin + (int64_t)Y * P + c0;
#pragma unroll
    for (int i = 0; i < TY; ++i) {
        if (!EDGE) {
            st4_nt(po + (int64_t)i * P, cur[i]);
        } else if (Y + i < N) {
            float* q = po + (int64_t)i * P;
            if (in3) {
                st4_nt(q, cur[i]);
            } else {
                if (in0) q[0] = cur[i].x;
                if (in1) q[1] = cur[i].y;
                if (in2) q[2] = cur[i].z;
            }
        }
    }
    return m;
}

template <int TY, bool CHK, bool FAST>
__global__ __launch_bounds__(256) void k_async_wide(const float* __restrict__ uin, const float* __restrict__ bin,
                                                    float* __restrict__ uout, StepArgs a, int tx, int D) {
    if (a.sc->stop) return;  // a previous check already stopped the step
    const int N = a.g.N;
    const int sx = (N + kWideStrip - 1) / kWideStrip, sy = (N + TY - 1) / TY;
    const int wid = xcd_logical_block(blockIdx.x, gridDim.x) * 4 + (int)(threadIdx.x >> 6);
    uint32_t m = 0;
    if (wid < sx * sy) {
        const int X = (wid % sx) * kWideStrip, Y = (wid / sx) * TY;
        if (X + kWideStrip <= N && Y + TY <= N)
            m = async_wide_strip<TY, false, CHK, FAST>(uin, bin, uout, a, tx, D, X, Y);
        else
            m = async_wide_strip<TY, true, CHK, FAST>(uin, bin, uout, a, tx, D, X, Y);
    }
    if (CHK) store_block_max<4>(m, a.sc, blockIdx.x);
}

template <int TY>
static void launch_wide_t(const float* uin, const float* b, float* uout, int tx, int D, bool check,
                          const StepArgs& a, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    if (check) {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async_wide<TY, true, true>), grid, block, 0, s, uin, b, uout, a, tx, D);
        else
            hipLaunchKernelGGL((k_async_wide<TY, true, false>), grid, block, 0, s, uin, b, uout, a, tx, D);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async_wide<TY, false, true>), grid, block, 0, s, uin, b, uout, a, tx, D);
        else
            hipLaunchKernelGGL((k_async_wide<TY, false, false>), grid, block, 0, s, uin, b, uout, a, tx, D);
    }
}

int64_t async_blocks(int N, int tx, int ty, int o) {
    if (async_wide_form(N, tx, ty, o)) {
        const int64_t strips = (int64_t)((N + kWideStrip - 1) / kWideStrip) * ((N + ty - 1) / ty);
        return ((strips + 3) / 4 + 7) / 8 * 8;
    }
    if (async_wave_form(tx, ty, o)) {
        const int64_t strips = (int64_t)((N + kWaveStrip - 1) / kWaveStrip) * ((N + ty - 1) / ty);
        return ((strips + 3) / 4 + 7) / 8 * 8;
    }
    const int64_t tiles = (int64_t)((N + tx - 1) / tx) * ((N + ty - 1) / ty);
    return (tiles + 7) / 8 * 8;
}

template <int TY>
static void launch_wave_t(const float* uin, const float* b, float* uout, int tx, int D, bool check,
                          const StepArgs& a, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    if (check) {
        if constexpr (TY % 8 == 0) {
            // a check far from the stop: the residual on every 8th row (strips start on one)
            if (a.fastdiv && a.smask[0] == 7 && D <= 8) {
                hipLaunchKernelGGL((k_async_wave<TY, true, true, true>), grid, block, 0, s, uin, b, uout, a, tx, D);
                return;
            }
        }
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async_wave<TY, true, true>), grid, block, 0, s, uin, b, uout, a, tx, D);
        else
            hipLaunchKernelGGL((k_async_wave<TY, true, false>), grid, block, 0, s, uin, b, uout, a, tx, D);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async_wave<TY, false, true>), grid, block, 0, s, uin, b, uout, a, tx, D);
        else
            hipLaunchKernelGGL((k_async_wave<TY, false, false>), grid, block, 0, s, uin, b, uout, a, tx, D);
    }
}

hipError_t launch_async(const float* uin, const float* b, float* uout, int tx, int ty, int D, int o, bool check,
                        const StepArgs& a, hipStream_t s) {
    if (tx < 1 || ty < 1 || tx > 256 || ty > 256 || o < 0 || o > 64 ||
        (int64_t)(tx + 2 * o) * (ty + 2 * o) > kAsyncMaxPts)
        return hipErrorInvalidValue;
    const int64_t blocks = async_blocks(a.g.N, tx, ty, o);
    if (blocks > (int64_t)0x7fffffff) return hipErrorInvalidValue;
    if (async_wide_form(a.g.N, tx, ty, o)) {
        const dim3 grid((unsigned)blocks);
        switch (ty) {
            case 4: launch_wide_t<4>(uin, b, uout, tx, D, check, a, grid, s); break;
            default: launch_wide_t<8>(uin, b, uout, tx, D, check, a, grid, s); break;
        }
        return hipGetLastError();
    }
    if (async_wave_form(tx, ty, o)) {
        const dim3 grid((unsigned)blocks);
        switch (ty) {
            case 4: launch_wave_t<4>(uin, b, uout, tx, D, check, a, grid, s); break;
            case 8: launch_wave_t<8>(uin, b, uout, tx, D, check, a, grid, s); break;
            case 16: launch_wave_t<16>(uin, b, uout, tx, D, check, a, grid, s); break;
            default: launch_wave_t<32>(uin, b, uout, tx, D, check, a, grid, s); break;
        }
        return hipGetLastError();
    }
    const size_t lds = (size_t)2 * (tx + 2 * o + 2) * (ty + 2 * o + 2) * sizeof(float);
    const dim3 grid((unsigned)blocks), block(kAsyncThreads);
    if (check) {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async<true, true>), grid, block, lds, s, uin, b, uout, a, tx, ty, D, o);
        else
            hipLaunchKernelGGL((k_async<true, false>), grid, block, lds, s, uin, b, uout, a, tx, ty, D, o);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_async<false, true>), grid, block, lds, s, uin, b, uout, a, tx, ty, D, o);
        else
            hipLaunchKernelGGL((k_async<false, false>), grid, block, lds, s, uin, b, uout, a, tx, ty, D, o);
    }
    return hipGetLastError();
}

}  // namespace jac
