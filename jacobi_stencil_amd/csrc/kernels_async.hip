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
// Here: tiles of tile_x columns by tile_y rows start at unknown (0, 0), the
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
        float bb[kAsyncPerThread];
#pragma unroll
        for (int q = 0; q < kAsyncPerThread; ++q) {
            const int p = threadIdx.x + q * kAsyncThreads;
            bb[q] = 0.0f;
            if (p < npts) {
                const int i = p / w, j = p - (p / w) * w;
                bb[q] = bin[g.origin + (int64_t)(ey0 + i) * P + (ex0 + j)];
            }
        }
        __syncthreads();
        // a point of the region is one of the tile's own
        auto owned = [&](int i, int j) {
            return ey0 + i >= y0 && ey0 + i < y1 && ex0 + j >= x0 && ex0 + j < x1;
        };
        if (CHK) {
            // residual of u_k on the tile's own points (the halo is u_k too)
#pragma unroll
            for (int q = 0; q < kAsyncPerThread; ++q) {
                const int p = threadIdx.x + q * kAsyncThreads;
                if (p < npts) {
                    const int i = p / w, j = p - (p / w) * w;
                    if (owned(i, j)) {
                        const int c = (i + 1) * lp + (j + 1);
                        const uint32_t v =
                            residual_bits(A[c], A[c + 1], A[c - 1], A[c - lp], A[c + lp], bb[q], r);
                        m = m > v ? m : v;
                    }
                }
            }
        }
        float* cur = A;
        float* nxt = B;
        for (int s = 0; s < D; ++s) {
#pragma unroll
            for (int q = 0; q < kAsyncPerThread; ++q) {
                const int p = threadIdx.x + q * kAsyncThreads;
                if (p < npts) {
                    const int i = p / w, j = p - (p / w) * w;
                    const int c = (i + 1) * lp + (j + 1);
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
            const int p = threadIdx.x + q * kAsyncThreads;
            if (p < npts) {
                const int i = p / w, j = p - (p / w) * w;
                if (owned(i, j)) dst[(int64_t)i * P + j] = cur[(i + 1) * lp + (j + 1)];
            }
        }
    }
    if (CHK) store_block_max<kAsyncThreads / 64>(m, a.sc, blockIdx.x);
}

int64_t async_blocks(int N, int tx, int ty) {
    const int64_t tiles = (int64_t)((N + tx - 1) / tx) * ((N + ty - 1) / ty);
    return (tiles + 7) / 8 * 8;
}

hipError_t launch_async(const float* uin, const float* b, float* uout, int tx, int ty, int D, int o, bool check,
                        const StepArgs& a, hipStream_t s) {
    if (tx < 1 || ty < 1 || tx > 256 || ty > 256 || o < 0 || o > 64 ||
        (int64_t)(tx + 2 * o) * (ty + 2 * o) > kAsyncMaxPts)
        return hipErrorInvalidValue;
    const int64_t blocks = async_blocks(a.g.N, tx, ty);
    if (blocks > (int64_t)0x7fffffff) return hipErrorInvalidValue;
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
