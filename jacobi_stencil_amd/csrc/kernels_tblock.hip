// kernels_tblock.hip -- exact temporal blocking (kernel b): D synchronous
// sweeps per pass over memory, bitwise identical to D launches of the sync
// sweep.
//
// The technique (page "stencil-jacobian.vercel.app", section 02, the
// ghost-zone method of Meng & Skadron): a block loads its tile with a halo D
// cells wide and, in sweep s, updates only the points that are still exact
// (at least s cells inside the loaded edge); after D sweeps the tile's core
// holds exactly what D synchronous sweeps produce, at the price of redundant
// work in the halo.
//
// MI355X design (differs from the page's 2-D tile): one wavefront owns a
// 256-column window (64 lanes x 4 columns, one 16-byte load per row) whose
// central 256 - 2*Dp columns are its output (Dp = D rounded up to a multiple
// of 4, so every load stays 16-byte aligned), and streams down a band of H
// output rows plus D rows above and below.  Time is pipelined along the rows:
// when row j of u_k arrives, level 1 (u_{k+1}) is computed for row j-1,
// level 2 for row j-2, ..., level D for row j-D, which is stored.  Each level
// keeps only its last two rows in registers; the west/east neighbours of a
// lane's 4 columns come from the adjacent lanes by DPP lane shifts; b rows go
// through a per-wavefront ring in LDS (level t reads b of row j-t).  Only the
// columns are recomputed redundantly (256 / (256 - 2*Dp)) and the band's D
// extra rows on each side ((H + 2D) / H); the 2-D tile of the page pays both
// factors squared.  Values that leave the exact cone (the window's outer
// columns, the first rows of each level) are computed but never stored and
// never feed a stored value.
//
// Boundary: at every level the ghost ring keeps its fixed values -- row -1 is
// 100 on columns 0..N-1, row N and columns -1 and N are 0.  Wavefronts whose
// window or row range touches the ring re-impose them after each level; the
// others skip that work.
#include "jacobi_internal.h"

namespace jac {

// Lane i receives lane i-1's value (lane 0 receives 0): DPP wave_shr:1.
__device__ __forceinline__ float from_left(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xF, 0xF, true));
}
// Lane i receives lane i+1's value (lane 63 receives 0): DPP wave_shl:1.
__device__ __forceinline__ float from_right(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xF, 0xF, true));
}

struct TBLane {
    int c0;          // first of the lane's 4 columns
    bool in[4];      // column is an unknown (0 <= col < N)
    bool core[4];    // column is an unknown this wavefront stores
};

template <bool FAST>
__device__ __forceinline__ float4 level_update(const float4& up, const float4& mid, const float4& dn,
                                               const float4& bb, float r, float d, float y) {
    const float wl = from_left(mid.w);
    const float er = from_right(mid.x);
    float4 o;
    o.x = jacobi_update<FAST>(mid.y, wl, up.x, dn.x, bb.x, r, d, y);
    o.y = jacobi_update<FAST>(mid.z, mid.x, up.y, dn.y, bb.y, r, d, y);
    o.z = jacobi_update<FAST>(mid.w, mid.y, up.z, dn.z, bb.z, r, d, y);
    o.w = jacobi_update<FAST>(er, mid.z, up.w, dn.w, bb.w, r, d, y);
    return o;
}

__device__ __forceinline__ uint32_t level_residual(const float4& up, const float4& mid, const float4& dn,
                                                   const float4& bb, float r, const TBLane& L) {
    const float wl = from_left(mid.w);
    const float er = from_right(mid.x);
    uint32_t v0 = L.core[0] ? residual_bits(mid.x, mid.y, wl, up.x, dn.x, bb.x, r) : 0u;
    uint32_t v1 = L.core[1] ? residual_bits(mid.y, mid.z, mid.x, up.y, dn.y, bb.y, r) : 0u;
    uint32_t v2 = L.core[2] ? residual_bits(mid.z, mid.w, mid.y, up.z, dn.z, bb.z, r) : 0u;
    uint32_t v3 = L.core[3] ? residual_bits(mid.w, er, mid.z, up.w, dn.w, bb.w, r) : 0u;
    uint32_t a = v0 > v1 ? v0 : v1, b = v2 > v3 ? v2 : v3;
    return a > b ? a : b;
}

// Re-impose the ghost ring on a computed row i of any level >= 1.
__device__ __forceinline__ void impose_ring(float4& v, int i, int N, const TBLane& L) {
    if (i == -1) {
        v.x = L.in[0] ? kTop : 0.0f;
        v.y = L.in[1] ? kTop : 0.0f;
        v.z = L.in[2] ? kTop : 0.0f;
        v.w = L.in[3] ? kTop : 0.0f;
    } else if (i == N) {
        v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if (i >= 0 && i < N) {
        if (!L.in[0]) v.x = 0.0f;
        if (!L.in[1]) v.y = 0.0f;
        if (!L.in[2]) v.z = 0.0f;
        if (!L.in[3]) v.w = 0.0f;
    }
}

template <int D, bool CHK, bool EDGE, bool FAST>
__device__ __forceinline__ uint32_t tb_band(const float* __restrict__ uin, const float* __restrict__ bin,
                                            float* __restrict__ uout, const StepArgs& a, const TBLane& L,
                                            bool lane_loads, int y0, int last, float4 (*ring)[64]) {
    constexpr int R = D + 1;
    const int N = a.g.N, P = a.g.P;
    const float r = a.r, d = a.d, y = a.y;
    const int lane = threadIdx.x & 63;
    const int j0 = y0 - D, j1 = last + D;
    const float* pu = uin + a.g.origin + L.c0;
    const float* pb = bin + a.g.origin + L.c0;
    float* po = uout + a.g.origin + L.c0;
    const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    bool store_lane = L.core[0];

    float4 up[D], mid[D];
#pragma unroll
    for (int t = 0; t < D; ++t) { up[t] = zero; mid[t] = zero; }
    uint32_t m = 0;

    float4 nu = zero, nb = zero;
    if (lane_loads) {
        nu = *reinterpret_cast<const float4*>(pu + (int64_t)j0 * P);
        nb = *reinterpret_cast<const float4*>(pb + (int64_t)j0 * P);
    }
    int s = 0;  // ring slot of row j
    for (int j = j0; j <= j1; ++j) {
        const float4 cur = nu;
        const float4 cb = nb;
        if (lane_loads && j < j1) {  // fetch the next row while this one is worked on
            nu = *reinterpret_cast<const float4*>(pu + (int64_t)(j + 1) * P);
            nb = *reinterpret_cast<const float4*>(pb + (int64_t)(j + 1) * P);
        }
        ring[s][lane] = cb;
        float4 nw = cur;  // level 0, row j
#pragma unroll
        for (int t = 1; t <= D; ++t) {
            int st = s - t;
            if (st < 0) st += R;
            const float4 bb = ring[st][lane];
            if (CHK && t == 1) {
                // residual of u_k on row j-1, from the same stencil level 1 reads
                const int i = j - 1;
                if (i >= y0 && i <= last) {
                    uint32_t v = level_residual(up[0], mid[0], nw, bb, r, L);
                    m = m > v ? m : v;
                }
            }
            float4 v = level_update<FAST>(up[t - 1], mid[t - 1], nw, bb, r, d, y);
            if (EDGE) impose_ring(v, j - t, N, L);
            up[t - 1] = mid[t - 1];
            mid[t - 1] = nw;
            nw = v;
        }
        const int i = j - D;
        if (i >= y0 && i <= last && store_lane) {
            float* q = po + (int64_t)i * P;
            if (L.core[3]) {
                *reinterpret_cast<float4*>(q) = nw;
            } else {
                q[0] = nw.x;
                if (L.core[1]) q[1] = nw.y;
                if (L.core[2]) q[2] = nw.z;
            }
        }
        s = (s + 1 == R) ? 0 : s + 1;
    }
    return m;
}

template <int D, bool CHK, bool FAST>
__global__ __launch_bounds__(64) void k_tblock(const float* __restrict__ uin, const float* __restrict__ bin,
                                               float* __restrict__ uout, StepArgs a, int H) {
    constexpr int Dp = (D + 3) & ~3;
    constexpr int Wout = 256 - 2 * Dp;
    __shared__ float4 ring[D + 1][64];
    if (a.sc->stop) return;  // a previous check already stopped the step
    const int N = a.g.N;
    const int lane = threadIdx.x;
    const int strips = (N + Wout - 1) / Wout;
    const int bands = (N + H - 1) / H;
    const int t = xcd_logical_block(blockIdx.x, gridDim.x);
    uint32_t m = 0;
    if (t < strips * bands) {
        const int x0 = (t % strips) * Wout;  // first output column
        const int X = x0 - Dp;               // first column of the window
        const int y0 = (t / strips) * H;
        const int last = (y0 + H < N ? y0 + H : N) - 1;
        TBLane L;
        L.c0 = X + 4 * lane;
        const bool core_lane = lane >= Dp / 4 && lane < 64 - Dp / 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            L.in[c] = L.c0 + c >= 0 && L.c0 + c < N;
            L.core[c] = core_lane && L.in[c];
        }
        // lanes wholly outside [0, N) would load only zero padding and the zero
        // ghost columns: they skip the loads and keep zeros
        const bool lane_loads = L.c0 < N && L.c0 + 4 > 0;
        const bool edge = X < 0 || X + 256 > N || y0 - D < 0 || last + D >= N;
        if (edge)
            m = tb_band<D, CHK, true, FAST>(uin, bin, uout, a, L, lane_loads, y0, last, ring);
        else
            m = tb_band<D, CHK, false, FAST>(uin, bin, uout, a, L, lane_loads, y0, last, ring);
    }
    if (CHK) store_block_max<1>(m, a.sc, blockIdx.x);
}

int tblock_rows(int N, int D) {
    // band height: long enough that the D extra rows above and below stay a
    // small fraction, short enough to give every SIMD several wavefronts
    (void)D;
    if (N >= 4096) return 128;
    if (N >= 1024) return 64;
    return 32;
}

int64_t tblock_blocks(int N, int D, int H) {
    const int Dp = (D + 3) & ~3;
    const int Wout = 256 - 2 * Dp;
    const int64_t tiles = (int64_t)((N + Wout - 1) / Wout) * ((N + H - 1) / H);
    return (tiles + 7) / 8 * 8;
}

template <int D>
static hipError_t launch_tb_d(const float* uin, const float* b, float* uout, bool check, const StepArgs& a,
                              int H, hipStream_t s) {
    constexpr int Dp = (D + 3) & ~3;
    constexpr int Wout = 256 - 2 * Dp;
    const int N = a.g.N;
    const int tiles = ((N + Wout - 1) / Wout) * ((N + H - 1) / H);
    const int blocks = (tiles + 7) / 8 * 8;
    if (check) {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_tblock<D, true, true>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H);
        else
            hipLaunchKernelGGL((k_tblock<D, true, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_tblock<D, false, true>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H);
        else
            hipLaunchKernelGGL((k_tblock<D, false, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H);
    }
    return hipGetLastError();
}

hipError_t launch_tblock(const float* uin, const float* b, float* uout, int D, bool check, const StepArgs& a,
                         int H, hipStream_t s) {
    if (H < 1) H = tblock_rows(a.g.N, D);
    switch (D) {
        case 1: return launch_tb_d<1>(uin, b, uout, check, a, H, s);
        case 2: return launch_tb_d<2>(uin, b, uout, check, a, H, s);
        case 3: return launch_tb_d<3>(uin, b, uout, check, a, H, s);
        case 4: return launch_tb_d<4>(uin, b, uout, check, a, H, s);
        case 5: return launch_tb_d<5>(uin, b, uout, check, a, H, s);
        case 6: return launch_tb_d<6>(uin, b, uout, check, a, H, s);
        case 7: return launch_tb_d<7>(uin, b, uout, check, a, H, s);
        case 8: return launch_tb_d<8>(uin, b, uout, check, a, H, s);
        case 9: return launch_tb_d<9>(uin, b, uout, check, a, H, s);
        case 10: return launch_tb_d<10>(uin, b, uout, check, a, H, s);
        case 11: return launch_tb_d<11>(uin, b, uout, check, a, H, s);
        case 12: return launch_tb_d<12>(uin, b, uout, check, a, H, s);
        case 13: return launch_tb_d<13>(uin, b, uout, check, a, H, s);
        case 14: return launch_tb_d<14>(uin, b, uout, check, a, H, s);
        case 15: return launch_tb_d<15>(uin, b, uout, check, a, H, s);
        case 16: return launch_tb_d<16>(uin, b, uout, check, a, H, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace jac
