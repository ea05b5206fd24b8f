// jacobi_internal.h -- geometry, scratch layout and device helpers shared by
// the HIP sources of libjacobi.  Not part of the public interface
// (include/jacobi.h is).
//
// The method (page "stencil-jacobian.vercel.app", sections 01 and 02): each
// backward-Euler step solves (1+4r) u - r (uE+uW+uN+uS) = b with b = u^n + dt*f,
// the top boundary at 100 and the other sides at 0, by point Jacobi until
// rho = ||b_A - A u||_inf / ||b_A||_inf < tol, checked every M sweeps.  Every
// kernel performs the same float32 operations in the same order, each rounded
// to nearest, none fused (the library is compiled with -ffp-contract=off):
//   sweep     S = ((uE + uW) + uN) + uS;  u' = (b + r*S) / d,  d = 1 + 4r
//   residual  e = (((uE-C) + (uW-C)) + (uN-C)) + (uS-C);  res = (b - C) + r*e
//   norm      bA = max |b + r*g|, g = 100 on the top row of unknowns, else 0
//   decision  rho = R / bA, R = max |res|; a step stops when !(rho >= tol)
//             (converged when rho < tol, failed when rho is NaN).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jac {

// ---------------------------------------------------------------- layout
//
// Every grid (u0, u1, b, s) is one "plane" of (N + 2*kPad) rows of pitch P
// floats.  Unknown (i, j) -- i the row from the top, j the column -- lives at
// origin + i*P + j with origin = kPad*P + kPad.  Row -1, row N, column -1 and
// column N are the ghost ring (top row 100 in u0/u1, everything else 0); the
// remaining padding is 0 and is never written after set-up.  kPad = 64 floats
// keeps column 0 of every row on a 256-byte boundary (P is a multiple of 64)
// and leaves room for halo loads of up to 63 cells beyond the ghost ring.
constexpr int kPad = 64;
constexpr float kTop = 100.0f;

struct Geom {
    int N;          // unknowns per side
    int P;          // row pitch in floats
    int64_t plane;  // floats per plane (multiple of 64)
    int64_t origin; // offset of unknown (0, 0)
};

inline Geom make_geom(int N) {
    Geom g;
    g.N = N;
    g.P = ((N + 2 * kPad) + 63) / 64 * 64;
    g.plane = (int64_t)g.P * (int64_t)(N + 2 * kPad);
    g.origin = (int64_t)kPad * g.P + kPad;
    return g;
}

// Device scratch (inside the caller's workspace, after the planes): a header
// and an array of per-block partial maxima.  A reduction kernel writes a
// partial per block with a plain store; a one-block kernel that runs next
// reduces them.  (One atomic per block on a shared word serialises at the
// memory side: thousands of blocks cost hundreds of microseconds.)
struct Scratch {
    uint32_t bA_bits;  // ||b_A||_inf of the current step
    uint32_t stop;     // 1 once a check of the current step has decided to stop
    uint32_t div_bad;  // inputs on which the constant-divisor quotient missed (set-up check)
    uint32_t check_seq;  // checks reduced so far in this step (the mailbox slot of the next)
    uint32_t pad0[12];
    // grid barrier of the persistent kernel (cleared before each launch), each
    // word on its own 64-byte line
    uint32_t bar_release;  // generation block 0 has released
    uint32_t pad1[15];
    uint32_t bar_unused;
    uint32_t pad2[15];
    uint32_t bar_error;    // set when a barrier wait timed out; every block then leaves
    uint32_t pad3[15];
    // followed by uint32_t partial[npart_cap]
};
static_assert(sizeof(Scratch) == 256, "scratch header is 256 bytes");

// Persistent-kernel barrier flags: one 128-byte line per block, after the header.
constexpr int kMaxPersistBlocks = 2048;
constexpr int kFlagStride = 32;  // uint32 words per flag line
__host__ __device__ inline uint32_t* scratch_flags(Scratch* sc) { return reinterpret_cast<uint32_t*>(sc + 1); }
__host__ __device__ inline uint32_t* scratch_partials(Scratch* sc) {
    return scratch_flags(sc) + (size_t)kMaxPersistBlocks * kFlagStride;
}

// Partial-maximum slots a context of size N reserves; every kernel that writes
// partials is launched with at most this many blocks (checked on the host).
inline int64_t partial_cap(int N) { return (int64_t)N * N / 64 + 65536; }

// Workspace after the partial slots (256-byte aligned): the edge-exchange words
// of the persistent kernel's resident tiles, 64 bits each.  min(5 Mi, 5 (N+31)^2)
// words: a tile of side T with halo depth H takes 8 H T words, at most 4.25
// per cell for T >= 32 and H <= 17, and one round holds at most 512 tiles of
// 64 x 64 (8704 words each).
inline int64_t exchange_words_cap(int N) {
    const int64_t a = 5 * (int64_t)(N + 31) * (N + 31);
    return a < ((int64_t)5 << 20) ? a : ((int64_t)5 << 20);
}
inline int64_t exchange_offset_floats(const Geom& g, int64_t npart_cap) {
    const int64_t end = 4 * g.plane + (int64_t)(sizeof(Scratch) / 4) + (int64_t)kMaxPersistBlocks * kFlagStride + npart_cap;
    return (end + 63) / 64 * 64;
}

// Host-visible results, in coherent pinned host memory that the device writes
// directly with system-scope stores (not held in its caches), so the host sees
// them without a system-wide cache flush behind every check.
constexpr int kRing = 64;   // check results kept in flight
constexpr uint32_t kEmpty = 0xFFFFFFFFu;  // never a |res| bit pattern (sign bit set)
struct Mailbox {
    uint32_t bA_bits;
    uint32_t pad[15];
    uint32_t R[kRing];
};

// Arguments every sweep-like kernel takes.
struct StepArgs {
    Geom g;
    float r, d, tol;
    float y;        // RN(1/d), for the constant-divisor quotient
    int fastdiv;    // 1: divide by the constant-divisor quotient (see div_d)
    Scratch* sc;
    Mailbox* mail;
    int slot;       // mailbox slot for this kernel's check; < 0: the device's check counter
    // temporal blocking deeper than 8: the levels whose residual a checking
    // launch measures (chk[0], and chk[1] or -1); its block maxima go to
    // partial slots [0, grid) and [grid, 2 grid)
    int chk[2];
    int force;         // 1: run even if a check has stopped the step (a redo)
    int64_t part_off;  // the reduction reads partial slots from here
    int slot2;         // >= 0: the reduction also reduces the next npart slots, a second check, into this
                       // mailbox slot (a launch that checks two levels)
    // per checked level, a row mask: a temporal-blocking launch measures the
    // residual on the rows i with (i & smask) == 0 only (0: every row).  Their
    // maximum is a lower bound of R, enough to show that a check goes on.
    int smask[2];
};

// ---------------------------------------------------------------- device

// n / d, rounded to nearest.  FAST uses the reciprocal y = RN(1/d) and one
// correction step (Markstein, "Computation of elementary functions on the IBM
// RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): q0 = RN(n*y),
// e = n - q0*d exactly by one fma, q = RN(q0 + e*y).  It has no special-case
// fixup, so it is not the IEEE quotient for n = +-Inf, NaN or -0 (Inf gives
// NaN, -0 gives +0).  A context uses FAST only (1) after a set-up kernel has
// found it equal to n / d on every other float n for its d, and (2) for work
// in which the host has shown that no numerator is Inf, NaN or -0.
template <bool FAST>
__device__ __forceinline__ float div_d(float n, float d, float y) {
    if constexpr (FAST) {
        const float q0 = n * y;
        const float e = __builtin_fmaf(-q0, d, n);
        return __builtin_fmaf(e, y, q0);
    } else {
        return n / d;
    }
}

template <bool FAST>
__device__ __forceinline__ float jacobi_update(float uE, float uW, float uN, float uS, float b, float r, float d,
                                               float y) {
    float S = uE + uW;
    S = S + uN;
    S = S + uS;
    float t = r * S;
    float n = b + t;
    return div_d<FAST>(n, d, y);
}

__device__ __forceinline__ uint32_t residual_bits(float C, float uE, float uW, float uN, float uS,
                                                  float b, float r) {
    float e = (uE - C) + (uW - C);
    e = e + (uN - C);
    e = e + (uS - C);
    float bc = b - C;
    float t = r * e;
    return __float_as_uint(fabsf(bc + t));  // NaN (any payload) sorts above +Inf
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
        v = v > w ? v : w;
    }
    return v;
}

// Lane i receives lane i-1's value (lane 0 receives 0): DPP wave_shr:1.
// A shift reads the source lane only if that lane is active (else 0): call it
// with every lane active -- `c ? x : from_left(v)` evaluates the shift only in
// the lanes without c; compute the shift first, then select.
__device__ __forceinline__ float from_left(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xF, 0xF, true));
}
// Lane i receives lane i+1's value (lane 63 receives 0): DPP wave_shl:1.
__device__ __forceinline__ float from_right(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xF, 0xF, true));
}

// 16-byte loads and stores; _nt marks them nontemporal (streamed data that
// this kernel reads or writes once: keeps it from displacing reused lines).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4_nt(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4_nt(float* p, const float4& v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}

// Buffer accesses through a raw resource descriptor (stride 0).  The hardware
// range-checks every lane's offset: a lane whose offset is kOOB loads zeros and
// its stores are dropped.  A loop can then issue the same memory instructions
// on every path -- lanes or rows that must not touch memory are masked by their
// offset rather than by a branch -- so the wait before a loaded value is used
// counts only the instructions issued after that load, not every store too.
// In-range offsets (voffset + soffset) must stay below kOOB = 2 GiB.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit data format, the gfx9 raw-buffer setting
constexpr int kAuxNT = 2;                    // nontemporal (streaming) cache policy
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)kOOB, kRawBufferWord3);
}
__device__ __forceinline__ float4 bld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void bst4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, const float4& v) {
    const f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r, (int)voff, (int)soff, kAuxNT);
}
__device__ __forceinline__ void bst1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}

// Blocks are handed to the 8 XCDs round-robin; give each XCD a contiguous
// range of logical tiles so that vertically adjacent tiles (which share halo
// rows) sit behind the same L2.  nblocks must be a multiple of 8; logical ids
// beyond the tile count are idle blocks.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
    int per = nblocks >> 3;
    return (b & 7) * per + (b >> 3);
}

__device__ __forceinline__ bool stop_set(const Scratch* sc) {
    return __atomic_load_n(&sc->stop, __ATOMIC_RELAXED) != 0;
}

// Block-wide max of `m` stored to the block's partial slot.  Every block of a
// reducing launch calls this exactly once (idle blocks with m = 0).
template <int WAVES>
__device__ __forceinline__ void store_block_max(uint32_t m, Scratch* sc, int64_t slot) {
    __shared__ uint32_t part[WAVES];
    m = wave_max_u32(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (WAVES == 1) {
        if (lane == 0) scratch_partials(sc)[slot] = m;
        return;
    }
    if (lane == 0) part[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t bm = part[0];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) bm = bm > part[w] ? bm : part[w];
        scratch_partials(sc)[slot] = bm;
    }
}

// ---------------------------------------------------------------- host side

// Launchers (kernels_*.hip).  All return hipSuccess or the launch error.
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);
hipError_t launch_ghosts(float* u, const Geom& g, hipStream_t s);
// b = u^n + s and the per-block norm partials; keep_u: the plane gets u^n.
hipError_t launch_rhs(const float* u, const float* src, float* b, bool keep_u, const StepArgs& a, hipStream_t s);
// Count the float inputs n (all 2^32 except Inf, NaN and -0) on which
// div_d<true> differs from n / d into sc->div_bad.
hipError_t launch_verify_div(float d, float y, Scratch* sc, hipStream_t s);
// Reduce npart partials.  norm: they are |b_A| maxima -- publish ||b_A||, clear
// the stop flag and the check counter.  Otherwise they are |res| maxima of a
// check -- unless the step has already stopped, publish R in mailbox slot
// a.slot (a.slot < 0: slot check_seq % kRing), count the check, and set the
// stop flag when !(R / ||b_A|| >= tol).
hipError_t launch_reduce(int64_t npart, bool norm, const StepArgs& a, hipStream_t s);
// Bandwidth probe: kind 0 copy (c = a), kind 1 add (c = a + b); n floats.
hipError_t launch_probe(float* c, const float* a, const float* b, int64_t n, int kind, bool nontemporal,
                        int blocks, hipStream_t s);
// Blocks each launch will use (for the host's partial-slot check).
int64_t rhs_blocks(int N);
int64_t sync_blocks(int N, int rows);
// Rows per wavefront of the synchronous sweep on a device with `cus` CUs.
int sync_rows_for(int N, int cus);
int64_t tblock_blocks(int N, int D, int H);
int tblock_max_rows(int N, int D);
int64_t async_blocks(int N, int tx, int ty, int o);
// The whole solve of nsteps steps in one cooperative kernel (see
// kernels_persist.hip).  `out` is pinned host memory for nsteps records of
// persist_out_bytes() each; `partial` needs 4 x grid slots; `xchg` holds
// xchg_words 64-bit words for the resident tiles' edge exchange.
hipError_t launch_persist(const StepArgs& sa, float* u0, float* u1, float* b, const float* s, uint32_t* partial,
                          uint64_t* xchg, int64_t xchg_words, void* out, int nsteps, int cur0, bool async_mode, int D,
                          int L, int tile_x, int tile_y, int side, int64_t max_sweeps, int cus, int* grid_used,
                          hipStream_t stream);
size_t persist_out_bytes();
// Block-asynchronous launch: tiles tx x ty (each 1..256), each worked on
// widened by o overlap cells per side ((tx+2o)*(ty+2o) <= 4096, o <= 64), a
// frozen one-cell halo around that, D in-tile sweeps.
hipError_t launch_async(const float* uin, const float* b, float* uout, int tx, int ty, int D, int o, bool check,
                        const StepArgs& a, hipStream_t s);
// Automatic band height on `cus` CUs that each hold `waves_per_cu` wavefronts
// of this depth.
int tblock_rows(int N, int D, int cus, int waves_per_cu);
int tblock_waves_per_cu(int D, bool fast);
// One synchronous sweep.  src != NULL: the unfused form, b holds u^n and
// b = u^n + src is formed per point.
hipError_t launch_sync(const float* uin, const float* b, const float* src, float* uout, bool check, int rows,
                       const StepArgs& a, hipStream_t s);
hipError_t launch_residual(const float* u, const float* b, const float* src, int rows, const StepArgs& a,
                           hipStream_t s);
// D sweeps (1..16) in one pass; H = output rows per wavefront band (>= 1).
// The first launch of a step that also forms b = u^n + s from u and src (the
// constant-divisor quotient only), stores b and leaves per-block maxima of
// |b_A| in the partial slots.
hipError_t launch_tblock_rhs(const float* u, const float* src, float* b, float* uout, int D, const StepArgs& a,
                             int H, hipStream_t s);
hipError_t launch_tblock(const float* uin, const float* b, float* uout, int D, bool check, const StepArgs& a,
                         int H, hipStream_t s);

}  // namespace jac
