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
// of 4, so every load stays 16-byte aligned), and streams along a band of H
// output rows plus D rows above and below (downwards, or for every other band
// from D = 5 on upwards).  Time is pipelined along the rows: when row j of u_k
// arrives, level 1 (u_{k+1}) is computed for the row before it, level 2 for
// the one before that, ..., level D for the row D back, which is stored.  Each level
// keeps only its last two rows in registers; the west/east neighbours of a
// lane's 4 columns come from the adjacent lanes by DPP lane shifts; b rows go
// through a per-wavefront ring in LDS (level t reads b of the row t back).  Only the
// columns are recomputed redundantly (256 / (256 - 2*Dp)) and the band's D
// extra rows on each side ((H + 2D) / H); the 2-D tile of the page pays both
// factors squared.  Values that leave the exact cone (the window's outer
// columns, the first rows of each level) are computed but never stored and
// never feed a stored value.
//
// The first launch of a time step may also form the right-hand side (RHS): it
// reads s where the others read b, takes b = u^n + s for every row it streams
// (one addition, as the separate right-hand-side pass does), stores b for its
// own rows and columns, and leaves per-block maxima of |b_A| for the norm.
//
// Boundary: at every level the ghost ring keeps its fixed values -- row -1 is
// 100 on columns 0..N-1, row N and columns -1 and N are 0.  Wavefronts whose
// window or row range touches the ring re-impose them after each level; the
// others skip that work.
#include "jacobi_internal.h"

#include <algorithm>
#include <type_traits>

namespace jac {

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

// Edge kinds of a wavefront band: interior; rows (the band's rows reach the
// ghost rows -1 or N, its window stays inside the grid); rows and columns (the
// window reaches past the grid, so the ghost columns -1 and N are re-imposed).
enum { kEdgeNone = 0, kEdgeRows = 1, kEdgeCols = 2 };

// Re-impose the ghost ring on a computed row i of any level >= 1.
template <int EK>
__device__ __forceinline__ void impose_ring(float4& v, int i, int N, const TBLane& L) {
    if (i == -1) {
        v.x = L.in[0] ? kTop : 0.0f;
        v.y = L.in[1] ? kTop : 0.0f;
        v.z = L.in[2] ? kTop : 0.0f;
        v.w = L.in[3] ? kTop : 0.0f;
    } else if (i == N) {
        v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else if (EK == kEdgeCols && i >= 0 && i < N) {
        if (!L.in[0]) v.x = 0.0f;
        if (!L.in[1]) v.y = 0.0f;
        if (!L.in[2]) v.z = 0.0f;
        if (!L.in[3]) v.w = 0.0f;
    }
}

// Column strips of the wavefront windows (window = 256 columns from X, core =
// the columns [x0, x1) it stores).  General layout: cores of Wout = 256 - 2Dp
// columns from column 0, each window Dp wider on both sides, so the first and
// last windows reach past the grid and re-impose the ghost columns every level.
// Aligned layout (N a multiple of 4 and N >= 256): the first window starts at
// column 0 and the last ends at column N - 1, so no window reaches past the
// grid -- the west neighbour of lane 0 and the east neighbour of lane 63, which
// the DPP shifts fill with 0, are then exactly the ghost columns.  Cores
// [0, 256 - Dp), then Wout wide, and the last window's [.., N); at N = 256 one
// window is the grid.
struct TBStrip {
    int X, x0, x1;
};

__host__ __device__ inline bool tb_aligned(int N) { return N % 4 == 0 && N >= 256; }

__host__ __device__ inline int tb_strip_count(int N, int Dp) {
    const int Wout = 256 - 2 * Dp;
    if (!tb_aligned(N)) return (N + Wout - 1) / Wout;
    if (N == 256) return 1;
    const int rest = N - 2 * (256 - Dp);
    return 2 + (rest > 0 ? (rest + Wout - 1) / Wout : 0);
}

__host__ __device__ inline TBStrip tb_strip(int N, int Dp, int s, int strips) {
    const int Wout = 256 - 2 * Dp;
    const int F = 256 - Dp;
    TBStrip t;
    if (!tb_aligned(N)) {
        t.x0 = s * Wout;
        t.x1 = t.x0 + Wout < N ? t.x0 + Wout : N;
        t.X = t.x0 - Dp;
    } else if (N == 256) {
        t.X = 0;
        t.x0 = 0;
        t.x1 = 256;
    } else if (s == 0) {
        t.X = 0;
        t.x0 = 0;
        t.x1 = F;
    } else {
        t.x0 = F + (s - 1) * Wout;
        if (s == strips - 1) {  // right-aligned; x0 >= N - 256 + Dp by the strip count
            t.X = N - 256;
            t.x1 = N;
        } else {
            t.X = t.x0 - Dp;
            t.x1 = t.x0 + Wout;
        }
    }
    return t;
}

// Row I/O of a wavefront's band, in one of two forms chosen by depth (both
// measured at 8192^2; the choice changes no result).
//
// TBGlobalIO: flat loads and stores; lanes and rows that must not touch memory
// skip them by a branch; nontemporal loads.  Fastest for the shallow depths,
// which are bound by memory bandwidth.
//
// TBBufferIO: buffer loads and stores issued on every row; a lane outside the
// grid, a column that is not stored or a row outside the band's output is
// masked by an out-of-range offset.  The memory instructions in flight are then
// the same on every path, so the wait for the prefetched row does not also wait
// for the row just stored; loads go through the caches normally, so the halo
// rows and columns that neighbouring bands re-read can hit in L2.  Fastest for
// the deep depths, which are bound by the arithmetic.
struct TBGlobalIO {
    const float* pu;
    const float* pb;
    float* po;
    float* pbo;
    int P;
    bool lane_loads, store_lane;

    __device__ __forceinline__ void init(const float* uin, const float* bin, float* uout, float* bout,
                                         const StepArgs& a, const TBLane& L, int X, bool loads, int j0, int y0) {
        (void)X;
        (void)j0;
        (void)y0;
        P = a.g.P;
        pu = uin + a.g.origin + L.c0;
        pb = bin + a.g.origin + L.c0;
        po = uout + a.g.origin + L.c0;
        pbo = bout ? bout + a.g.origin + L.c0 : nullptr;
        lane_loads = loads;
        store_lane = L.core[0];
    }
    // row j of u_k and b into (nu, nb); rows outside [j0, j1] are not needed
    __device__ __forceinline__ void load(float4& nu, float4& nb, int j, int j0, int j1) {
        if (lane_loads && j >= j0 && j <= j1) {
            nu = ld4_nt(pu + (int64_t)j * P);
            nb = ld4_nt(pb + (int64_t)j * P);
        }
    }
    template <bool EDGE>
    __device__ __forceinline__ void store_to(float* base, const float4& out, int i, bool row_out, const TBLane& L) {
        if (row_out && store_lane) {
            float* q = base + (int64_t)i * P;
            if (L.core[3]) {
                st4_nt(q, out);
            } else {
                q[0] = out.x;
                if (L.core[1]) q[1] = out.y;
                if (L.core[2]) q[2] = out.z;
            }
        }
    }
    template <bool EDGE>
    __device__ __forceinline__ void store(const float4& out, int i, bool row_out, int y0, const TBLane& L) {
        (void)y0;
        store_to<EDGE>(po, out, i, row_out, L);
    }
    // row j of b (RHS launches)
    template <bool EDGE>
    __device__ __forceinline__ void store_b(const float4& v, int j, bool row_out, int y0, const TBLane& L) {
        (void)y0;
        store_to<EDGE>(pbo, v, j, row_out, L);
    }
};

struct TBBufferIO {
    __amdgpu_buffer_rsrc_t ru, rb;  // u_k and b, from row j0 - 1 and window column X
    __amdgpu_buffer_rsrc_t ro;      // output, from row y0 and window column X
    __amdgpu_buffer_rsrc_t rbo;     // b output of an RHS launch, from row y0 and window column X
    uint32_t vload;                 // the lane's byte offset in a row; kOOB: lane wholly outside [0, N)
    uint32_t vst4;                  // 16-byte store offset of a lane whose 4 columns are all stored
    uint32_t vst1[4];               // dword store offsets of a partly stored lane's columns (EDGE)
    uint32_t rowb;                  // row pitch in bytes

    __device__ __forceinline__ void init(const float* uin, const float* bin, float* uout, float* bout,
                                         const StepArgs& a, const TBLane& L, int X, bool loads, int j0, int y0) {
        const int P = a.g.P;
        rowb = (uint32_t)P * 4u;
        ru = make_rsrc(uin + a.g.origin + (int64_t)(j0 - 1) * P + X);
        rb = make_rsrc(bin + a.g.origin + (int64_t)(j0 - 1) * P + X);
        ro = make_rsrc(uout + a.g.origin + (int64_t)y0 * P + X);
        if (bout) rbo = make_rsrc(bout + a.g.origin + (int64_t)y0 * P + X);
        const uint32_t lb = (uint32_t)(threadIdx.x & 63) * 16u;
        vload = loads ? lb : kOOB;
        const bool full = L.core[0] && L.core[1] && L.core[2] && L.core[3];
        vst4 = full ? lb : kOOB;
#pragma unroll
        for (int c = 0; c < 4; ++c) vst1[c] = (!full && L.core[c]) ? lb + 4u * c : kOOB;
    }
    // row j of u_k and b into (nu, nb); the row one past the band's end
    // (j0 - 1 or j1 + 1, in the direction of travel) lies inside the padded
    // plane and is loaded and left unused
    __device__ __forceinline__ void load(float4& nu, float4& nb, int j, int j0, int j1) {
        (void)j1;
        const uint32_t so = (uint32_t)(j - j0 + 1) * rowb;
        nu = bld4(ru, vload, so);
        nb = bld4(rb, vload, so);
    }
    template <bool EDGE>
    __device__ __forceinline__ void store_to(__amdgpu_buffer_rsrc_t r, const float4& out, int i, bool row_out,
                                             int y0) {
        const uint32_t so = row_out ? (uint32_t)(i - y0) * rowb : 0u;
        bst4_nt(r, row_out ? vst4 : kOOB, so, out);
        if (EDGE) {
            bst1(r, row_out ? vst1[0] : kOOB, so, out.x);
            bst1(r, row_out ? vst1[1] : kOOB, so, out.y);
            bst1(r, row_out ? vst1[2] : kOOB, so, out.z);
            bst1(r, row_out ? vst1[3] : kOOB, so, out.w);
        }
    }
    template <bool EDGE>
    __device__ __forceinline__ void store(const float4& out, int i, bool row_out, int y0, const TBLane& L) {
        (void)L;
        store_to<EDGE>(ro, out, i, row_out, y0);
    }
    // row j of b (RHS launches)
    template <bool EDGE>
    __device__ __forceinline__ void store_b(const float4& v, int j, bool row_out, int y0, const TBLane& L) {
        (void)L;
        store_to<EDGE>(rbo, v, j, row_out, y0);
    }
};

template <int D>
using TBIO = typename std::conditional<(D >= 5), TBBufferIO, TBGlobalIO>::type;

// The streaming state of one wavefront: for every level t < D three row
// registers whose roles rotate (old = the row before, mid, new = the row after,
// in the direction of travel, as seen by level t+1), the prefetched next row,
// the ring slot.  RHS: the b operand holds s and b = u^n + s is formed per row
// (CHK and RHS never go together).  DIR = +1 streams the band downwards, -1 upwards; going up,
// the "before" rows lie below, so the update and the residual are handed the
// old and new rows as south and north instead of north and south -- every
// point sees the same neighbours in the same order either way.
template <int D, bool CHK, int EK, bool FAST, int DIR, bool RHS, int CL>
struct TBStream {
    TBIO<D> io;
    float r, d, y;
    int N, j0, j1, y0, last;
    TBLane L;
    float4 (*ring)[64];
    float4 nu, nb;  // row j+1 of u_k and b, loaded one row ahead
    int s;          // ring slot of the current row
    uint32_t m;     // running max |res| (CHK) or |b_A| (RHS), as bits
    uint32_t m2;    // D >= 9: running max |res| of the second checked level
    int chk0, chk1; // D >= 9: the checked levels (chk1 < 0: one)
    int sm0, sm1;   // their row masks: the residual is taken on rows i with (i & mask) == 0

    // One row j: read it, push every level one row further, store level D.
    // UP/MID/NEW are the level registers in this row's rotation.
    __device__ __forceinline__ void row(int j, float4 (&UP)[D], float4 (&MID)[D], float4 (&NEW)[D]) {
        constexpr int R = D + 1;
        const int lane = threadIdx.x & 63;
        NEW[0] = nu;
        const float4 cb = RHS ? make_float4(nu.x + nb.x, nu.y + nb.y, nu.z + nb.z, nu.w + nb.w) : nb;
        io.load(nu, nb, j + DIR, j0, j1);  // fetch the next row while this one is worked on
        ring[s][lane] = cb;
        if (RHS) {
            // b of an own row is stored once, by the wavefront whose core holds it;
            // ||b_A|| = max |b + r*g| with g = 100 on row 0
            const bool own = j >= y0 && j <= last;
            io.template store_b<EK == kEdgeCols>(cb, j, own, y0, L);
            if (own) {
                const float rg = r * (j == 0 ? kTop : 0.0f);
                const uint32_t v0 = L.core[0] ? __float_as_uint(fabsf(cb.x + rg)) : 0u;
                const uint32_t v1 = L.core[1] ? __float_as_uint(fabsf(cb.y + rg)) : 0u;
                const uint32_t v2 = L.core[2] ? __float_as_uint(fabsf(cb.z + rg)) : 0u;
                const uint32_t v3 = L.core[3] ? __float_as_uint(fabsf(cb.w + rg)) : 0u;
                const uint32_t x = v0 > v1 ? v0 : v1, z = v2 > v3 ? v2 : v3;
                const uint32_t w = x > z ? x : z;
                m = m > w ? m : w;
            }
        }
        float4 out;
        const int depth = DIR > 0 ? j - j0 : j1 - j;  // level t is exact from the (2t)-th row streamed on
        // b of the next level is read one level ahead, so the LDS latency
        // overlaps the current level's arithmetic
        // (two buffers by level parity, so no copies between them)
        auto slot = [&](int t) { return s - t < 0 ? s - t + R : s - t; };
        float4 bq[2];
        bq[1] = ring[slot(1)][lane];
#pragma unroll
        for (int t = 1; t <= D; ++t) {
            if (2 * t <= depth) {
                const float4 bb = bq[t & 1];
                if (t < D) bq[(t + 1) & 1] = ring[slot(t + 1)][lane];
                if constexpr (CHK && D >= 9) {
                    // residual of level t-1 where a check falls, on the row level t
                    // computes, from the stencil it reads: levels fixed at compile time
                    // (CL >= 0: C0 = CL & 15, C1 = (CL >> 4) - 1) or passed at run time
                    constexpr int C0 = CL >= 0 ? (CL & 15) : -1, C1 = CL >= 0 ? (CL >> 4) - 1 : -1;
                    const bool at0 = CL >= 0 ? (t - 1 == C0) : (t - 1 == chk0);
                    const bool at1 = CL >= 0 ? (t - 1 == C1) : (t - 1 == chk1);
                    if (at0 || at1) {
                        const int i = j - DIR * t;
                        if (i >= y0 && i <= last && (i & (at0 ? sm0 : sm1)) == 0) {
                            const uint32_t v = DIR > 0 ? level_residual(UP[t - 1], MID[t - 1], NEW[t - 1], bb, r, L)
                                                       : level_residual(NEW[t - 1], MID[t - 1], UP[t - 1], bb, r, L);
                            if (at0) m = m > v ? m : v;
                            else m2 = m2 > v ? m2 : v;
                        }
                    }
                } else if (CHK && t == 1) {
                    // residual of u_k on the row level 1 computes, from the stencil it reads
                    const int i = j - DIR;
                    if (i >= y0 && i <= last && (i & sm0) == 0) {
                        const uint32_t v = DIR > 0 ? level_residual(UP[0], MID[0], NEW[0], bb, r, L)
                                                   : level_residual(NEW[0], MID[0], UP[0], bb, r, L);
                        m = m > v ? m : v;
                    }
                }
                float4 v = DIR > 0 ? level_update<FAST>(UP[t - 1], MID[t - 1], NEW[t - 1], bb, r, d, y)
                                   : level_update<FAST>(NEW[t - 1], MID[t - 1], UP[t - 1], bb, r, d, y);
                if (EK != kEdgeNone) impose_ring<EK>(v, j - DIR * t, N, L);
                if (t < D) NEW[t] = v;
                else out = v;
            }
        }
        const int i = j - DIR * D;
        io.template store<EK == kEdgeCols>(out, i, i >= y0 && i <= last, y0, L);
        s = (s + 1 == R) ? 0 : s + 1;
    }
};

template <int D, bool CHK, int EK, bool FAST, int DIR, bool RHS, int CL>
__device__ __forceinline__ uint32_t tb_band(const float* __restrict__ uin, const float* __restrict__ bin,
                                            float* __restrict__ uout, float* __restrict__ bout, const StepArgs& a,
                                            const TBLane& L, int X, bool lane_loads, int y0, int last,
                                            float4 (*ring)[64], uint32_t& m2) {
    TBStream<D, CHK, EK, FAST, DIR, RHS, CL> st;
    st.N = a.g.N;
    st.r = a.r;
    st.d = a.d;
    st.y = a.y;
    st.j0 = y0 - D;
    st.j1 = last + D;
    st.y0 = y0;
    st.last = last;
    st.io.init(uin, bin, uout, bout, a, L, X, lane_loads, st.j0, y0);
    st.L = L;
    st.ring = ring;
    st.s = 0;
    st.m = 0;
    st.m2 = 0;
    st.chk0 = a.chk[0];
    st.chk1 = a.chk[1];
    st.sm0 = a.smask[0];
    st.sm1 = a.smask[1];
    const float4 zero = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    st.nu = zero;
    st.nb = zero;
    const int first = DIR > 0 ? st.j0 : st.j1;
    st.io.load(st.nu, st.nb, first, st.j0, st.j1);
    float4 A[D], B[D], C[D];
#pragma unroll
    for (int t = 0; t < D; ++t) { A[t] = zero; B[t] = zero; C[t] = zero; }
    // Issue priority by progress (D >= 5).  The SIMD's arbiter favours the
    // oldest wavefront, so of the three sharing a SIMD the first dispatched
    // finished a band at ~158 us, the last at ~215 us, running alone for its
    // final ~35 us, where one wavefront cannot keep the VALU busy.  Lowering
    // the priority in steps at 60, 85 and 97 % of the band lets the others
    // catch up before the end (8192^2, D = 8: 58.9 -> 57.5 ms per solve with
    // steps at 75/90/97 %, 0.5 % less again at 60/85/97; 2048^2: 9.21 ->
    // 8.69 ms).  The shallow, memory-bound depths gain nothing.  Only the
    // order of issue changes.
    const int total = st.j1 - st.j0 + 1;
    int level = -1;
    auto set_prio = [&](int done) {
        if constexpr (D < 5) return;
        const int p = 100 * done;
        const int l = p < 60 * total ? 0 : (p < 85 * total ? 1 : (p < 97 * total ? 2 : 3));
        if (l == level) return;
        level = l;
        if (l == 0) __builtin_amdgcn_s_setprio(3);
        else if (l == 1) __builtin_amdgcn_s_setprio(2);
        else if (l == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
    };
    // Three rows per trip, the level registers rotating A -> B -> C.  While
    // the pipeline fills (the first 2D rows of the band) a row computes only
    // the levels that are already exact.
    if constexpr (DIR > 0) {
        for (int j = st.j0; j <= st.j1; j += 3) {
            set_prio(j - st.j0);
            st.row(j, A, B, C);
            if (j + 1 > st.j1) break;
            st.row(j + 1, B, C, A);
            if (j + 2 > st.j1) break;
            st.row(j + 2, C, A, B);
        }
    } else {
        for (int j = st.j1; j >= st.j0; j -= 3) {
            set_prio(st.j1 - j);
            st.row(j, A, B, C);
            if (j - 1 < st.j0) break;
            st.row(j - 1, B, C, A);
            if (j - 2 < st.j0) break;
            st.row(j - 2, C, A, B);
        }
    }
    m2 = st.m2;
    return st.m;
}

template <int D, bool CHK, bool FAST, int DIR, bool RHS, int CL>
__device__ __forceinline__ uint32_t tb_band_kind(const float* __restrict__ uin, const float* __restrict__ bin,
                                                 float* __restrict__ uout, float* __restrict__ bout,
                                                 const StepArgs& a, const TBLane& L, int X, bool lane_loads, int y0,
                                                 int last, float4 (*ring)[64], bool cols, bool rows, uint32_t& m2) {
    if (cols)
        return tb_band<D, CHK, kEdgeCols, FAST, DIR, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring,
                                                          m2);
    if (rows)
        return tb_band<D, CHK, kEdgeRows, FAST, DIR, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring,
                                                          m2);
    return tb_band<D, CHK, kEdgeNone, FAST, DIR, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring,
                                                      m2);
}

// Register budget per depth: up to 4, four wavefronts per SIMD (128 VGPRs);
// 5..11 three (168 VGPRs: the launch sizes its bands for three wavefronts per
// SIMD anyway; the pipelines of 9..11 levels fit without spilling); deeper
// pipelines two.
template <int D>
constexpr int tb_waves_per_simd() { return D <= 4 ? 4 : (D <= 11 ? 3 : 2); }

// RHS (the first launch of a step): bin is s, bout receives b; it runs
// whatever the stop flag says, since the norm reduction after it clears the
// flag the previous step left set.  CL (D >= 9, CHK): the checked levels fixed
// at compile time (see TBStream::row), or -1 to take them from the arguments.
template <int D, bool CHK, bool FAST, bool RHS, int CL = -1>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(tb_waves_per_simd<D>())))
void k_tblock(const float* __restrict__ uin, const float* __restrict__ bin,
                                               float* __restrict__ uout, StepArgs a, int H,
                                               float* __restrict__ bout) {
    static_assert(!(CHK && RHS), "a launch either checks or forms b");
    constexpr int Dp = (D + 3) & ~3;
    __shared__ float4 ring[D + 1][64];
    if (!RHS && !a.force && a.sc->stop) return;  // a previous check already stopped the step
    const int N = a.g.N;
    const int lane = threadIdx.x;
    const int strips = tb_strip_count(N, Dp);
    const int bands = (N + H - 1) / H;
    const int t = xcd_logical_block(blockIdx.x, gridDim.x);
    uint32_t m = 0, m2 = 0;
    if (t < strips * bands) {
        const TBStrip sp = tb_strip(N, Dp, t % strips, strips);
        const int X = sp.X;                  // first column of the window
        const int y0 = (t / strips) * H;
        const int last = (y0 + H < N ? y0 + H : N) - 1;
        TBLane L;
        L.c0 = X + 4 * lane;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            L.in[c] = L.c0 + c >= 0 && L.c0 + c < N;
            L.core[c] = L.c0 + c >= sp.x0 && L.c0 + c < sp.x1;
        }
        // lanes wholly outside [0, N) would load only zero padding and the zero
        // ghost columns: they skip the loads and keep zeros
        const bool lane_loads = L.c0 < N && L.c0 + 4 > 0;
        const bool cols = X < 0 || X + 256 > N;
        const bool rows = y0 - D < 0 || last + D >= N;
        // From D = 5 odd bands stream upwards: two vertically adjacent bands
        // (behind the same L2) then read the rows they share -- each one's
        // halo is the other's edge -- at the same time, both at their start
        // or both at their end, instead of a whole band apart (D = 8 at
        // 8192^2: 635 -> 584 MB fetched per launch, 202 -> 197 us; D = 6: 200
        // -> 189 us).  The shallow depths keep one direction: their loads are
        // nontemporal, not kept in L2 for the neighbour, and alternating ran
        // slower (D = 4: 169 -> 182 us, D = 2: 169 -> 177 us).
        if constexpr (D >= 5) {
            if ((t / strips) & 1)
                m = tb_band_kind<D, CHK, FAST, -1, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring,
                                                        cols, rows, m2);
            else
                m = tb_band_kind<D, CHK, FAST, 1, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring,
                                                       cols, rows, m2);
        } else {
            m = tb_band_kind<D, CHK, FAST, 1, RHS, CL>(uin, bin, uout, bout, a, L, X, lane_loads, y0, last, ring, cols,
                                                   rows, m2);
        }
    }
    if (CHK || RHS) store_block_max<1>(m, a.sc, blockIdx.x);
    if (CHK && D >= 9) store_block_max<1>(m2, a.sc, (int64_t)gridDim.x + blockIdx.x);
}

// Resident wavefronts per CU for the checking variant of depth D (the one with
// the most registers), from the runtime's occupancy calculator.
template <int D, int CL = -1>
static int tb_waves_per_cu_cl(bool fast) {
    int n = 0;
    hipError_t e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tblock<D, true, true, false, CL>, 64, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tblock<D, true, false, false, CL>, 64, 0);
    return (e == hipSuccess && n > 0) ? n : 4;
}

// (of every checking kernel a launch of depth D may use: bands sized for more
// wavefronts than one of them holds would leave a second, partial round)
template <int D>
static int tb_waves_per_cu(bool fast) {
    int n = tb_waves_per_cu_cl<D>(fast);
    if constexpr (D == 11) {
        n = std::min(n, tb_waves_per_cu_cl<11, 0 | (9 << 4)>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 1 | (10 << 4)>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 2 | (11 << 4)>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 3>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 4>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 5>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 6>(fast));
        n = std::min(n, tb_waves_per_cu_cl<11, 7>(fast));
    }
    return n;
}

int tblock_waves_per_cu(int D, bool fast) {
    switch (D) {
        case 1: return tb_waves_per_cu<1>(fast);
        case 2: return tb_waves_per_cu<2>(fast);
        case 3: return tb_waves_per_cu<3>(fast);
        case 4: return tb_waves_per_cu<4>(fast);
        case 5: return tb_waves_per_cu<5>(fast);
        case 6: return tb_waves_per_cu<6>(fast);
        case 7: return tb_waves_per_cu<7>(fast);
        case 8: return tb_waves_per_cu<8>(fast);
        case 9: return tb_waves_per_cu<9>(fast);
        case 10: return tb_waves_per_cu<10>(fast);
        case 11: return tb_waves_per_cu<11>(fast);
        case 12: return tb_waves_per_cu<12>(fast);
        case 13: return tb_waves_per_cu<13>(fast);
        case 14: return tb_waves_per_cu<14>(fast);
        case 15: return tb_waves_per_cu<15>(fast);
        case 16: return tb_waves_per_cu<16>(fast);
        default: return 4;
    }
}

// Band height: the shortest bands (most parallelism) such that the whole grid
// is one round of resident wavefronts -- a second, partly filled round would
// leave most SIMDs idle at the end -- but at least 4 rows.  Small grids (N up to
// ~2048) hit the floor: there a launch is bound by the latency of a band's
// row pipeline, and short bands (many wavefronts, more recomputed rows) beat
// long ones (N = 256, D = 8: 6.2 ms per ten steps at 4 rows, 10.0 at 16).  Resident waves are
// counted at most four per SIMD: more only shortens the bands (more re-read
// rows) without adding issue slots the arithmetic needs.  For D = 5..8 (bound
// by the arithmetic) the round is sized for three per SIMD: the longer bands
// recompute fewer rows, which at 8192^2 outweighed a fourth wavefront (D = 8:
// 202 vs 212 us per launch, D = 6: 195 vs 207 us); deeper pipelines fit only
// two per SIMD and need both.  Depths up to 4 are bound by
// memory bandwidth: there bands of at most 64 rows (more wavefronts than one
// round, each shorter) measured up to 15% faster than the one-round height.
int tblock_rows(int N, int D, int cus, int waves_per_cu) {
    const int Dp = (D + 3) & ~3;
    const int strips = tb_strip_count(N, Dp);
    int w = waves_per_cu < 16 ? waves_per_cu : 16;
    if (D >= 5 && D <= 8 && w > 12) w = 12;
    const int resident_waves = cus * w;
    int bands = resident_waves / strips;
    if (bands < 1) bands = 1;
    int H = (N + bands - 1) / bands;
    if (D <= 4 && H > 64) H = 64;
    return H < 4 ? 4 : H;
}

// Buffer row I/O (D >= 5) addresses a band's rows by 32-bit byte offsets from
// the row before it, and offsets from kOOB (2 GiB) on read as zeros: a band's
// rows plus two on each side must span less than that.  Flat I/O (D <= 4) has
// no limit.
int tblock_max_rows(int N, int D) {
    if (D < 5) return INT32_MAX;
    const int64_t rowb = (int64_t)make_geom(N).P * 4;
    const int64_t h = ((int64_t)kOOB - 1024) / rowb - 2 * D - 4;
    return h < 1 ? 1 : (h > INT32_MAX ? INT32_MAX : (int)h);
}

int64_t tblock_blocks(int N, int D, int H) {
    const int Dp = (D + 3) & ~3;
    const int64_t tiles = (int64_t)tb_strip_count(N, Dp) * ((N + H - 1) / H);
    return (tiles + 7) / 8 * 8;
}

// Launches of 11 sweeps over checks every 8 (the deep driver's common case)
// run one of eight kernels with the checked levels fixed at compile time
// -- (0, 8), (1, 9), (2, 10), 3, 4, 5, 6, 7: every launch of that schedule --
// so no run-time test sits between the levels of the unrolled pipeline
// (8192^2: 249 -> ~224 us per launch).  Other levels take the general kernel.
template <int CL, bool FAST>
static void launch_tb11_cl(int blocks, const float* uin, const float* b, float* uout, const StepArgs& a, int H,
                           hipStream_t s) {
    float* none = nullptr;
    hipLaunchKernelGGL((k_tblock<11, true, FAST, false, CL>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H,
                       none);
}

template <bool FAST>
static bool launch_tb11_fixed(int blocks, const float* uin, const float* b, float* uout, const StepArgs& a, int H,
                              hipStream_t s) {
    const int c0 = a.chk[0], c1 = a.chk[1];
    if (c1 >= 0 && !(c1 == c0 + 8 && c0 <= 2)) return false;
    if (c1 < 0 && !(c0 >= 3 && c0 <= 7)) return false;
    switch (c0) {
        case 0: launch_tb11_cl<0 | (9 << 4), FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 1: launch_tb11_cl<1 | (10 << 4), FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 2: launch_tb11_cl<2 | (11 << 4), FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 3: launch_tb11_cl<3, FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 4: launch_tb11_cl<4, FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 5: launch_tb11_cl<5, FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 6: launch_tb11_cl<6, FAST>(blocks, uin, b, uout, a, H, s); return true;
        case 7: launch_tb11_cl<7, FAST>(blocks, uin, b, uout, a, H, s); return true;
        default: return false;
    }
}

template <int D>
static hipError_t launch_tb_d(const float* uin, const float* b, float* uout, bool check, const StepArgs& a,
                              int H, hipStream_t s) {
    const int blocks = (int)tblock_blocks(a.g.N, D, H);
    float* none = nullptr;
    if constexpr (D == 11) {
        if (check && (a.fastdiv ? launch_tb11_fixed<true>(blocks, uin, b, uout, a, H, s)
                                : launch_tb11_fixed<false>(blocks, uin, b, uout, a, H, s)))
            return hipGetLastError();
    }
    if (check) {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_tblock<D, true, true, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H,
                               none);
        else
            hipLaunchKernelGGL((k_tblock<D, true, false, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H,
                               none);
    } else {
        if (a.fastdiv)
            hipLaunchKernelGGL((k_tblock<D, false, true, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H,
                               none);
        else
            hipLaunchKernelGGL((k_tblock<D, false, false, false>), dim3(blocks), dim3(64), 0, s, uin, b, uout, a, H,
                               none);
    }
    return hipGetLastError();
}

// The right-hand-side variant exists for the constant-divisor quotient only;
// with the IEEE quotient the step keeps the separate right-hand-side pass.
template <int D>
static hipError_t launch_tb_rhs_d(const float* u, const float* src, float* b, float* uout, const StepArgs& a, int H,
                                  hipStream_t s) {
    if (!a.fastdiv) return hipErrorInvalidValue;
    const int blocks = (int)tblock_blocks(a.g.N, D, H);
    hipLaunchKernelGGL((k_tblock<D, false, true, true>), dim3(blocks), dim3(64), 0, s, u, src, uout, a, H, b);
    return hipGetLastError();
}

hipError_t launch_tblock_rhs(const float* u, const float* src, float* b, float* uout, int D, const StepArgs& a,
                             int H, hipStream_t s) {
    switch (D) {
        case 1: return launch_tb_rhs_d<1>(u, src, b, uout, a, H, s);
        case 2: return launch_tb_rhs_d<2>(u, src, b, uout, a, H, s);
        case 3: return launch_tb_rhs_d<3>(u, src, b, uout, a, H, s);
        case 4: return launch_tb_rhs_d<4>(u, src, b, uout, a, H, s);
        case 5: return launch_tb_rhs_d<5>(u, src, b, uout, a, H, s);
        case 6: return launch_tb_rhs_d<6>(u, src, b, uout, a, H, s);
        case 7: return launch_tb_rhs_d<7>(u, src, b, uout, a, H, s);
        case 8: return launch_tb_rhs_d<8>(u, src, b, uout, a, H, s);
        case 9: return launch_tb_rhs_d<9>(u, src, b, uout, a, H, s);
        case 10: return launch_tb_rhs_d<10>(u, src, b, uout, a, H, s);
        case 11: return launch_tb_rhs_d<11>(u, src, b, uout, a, H, s);
        case 12: return launch_tb_rhs_d<12>(u, src, b, uout, a, H, s);
        case 13: return launch_tb_rhs_d<13>(u, src, b, uout, a, H, s);
        case 14: return launch_tb_rhs_d<14>(u, src, b, uout, a, H, s);
        case 15: return launch_tb_rhs_d<15>(u, src, b, uout, a, H, s);
        case 16: return launch_tb_rhs_d<16>(u, src, b, uout, a, H, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tblock(const float* uin, const float* b, float* uout, int D, bool check, const StepArgs& a,
                         int H, hipStream_t s) {
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
