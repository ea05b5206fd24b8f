// kernels_probe.hip -- memory-bandwidth probes: the achievable-bandwidth
// reference the sweep kernels are measured against (the role of the
// bandwidth probe on page "cuda-solver-lab", "Hardware ceilings"), and a
// kernel of known traffic for calibrating the memory counters.
//
//   copy: c = a        (4 bytes read, 4 written per element)
//   add:  c = a + b    (8 read, 4 written: the mix of a sweep, which reads
//                       u_k and b and writes u_{k+1})
// 16-byte accesses, a grid of a few wavefronts per SIMD striding over the
// arrays; nontemporal stores on request.
#include "jacobi_internal.h"

namespace jac {

template <int KIND, bool NT>
__global__ __launch_bounds__(256) void k_probe(float4* __restrict__ c, const float4* __restrict__ a,
                                               const float4* __restrict__ b, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 v = a[i];
        if (KIND == 1) {
            const float4 w = b[i];
            v.x = v.x + w.x;
            v.y = v.y + w.y;
            v.z = v.z + w.z;
            v.w = v.w + w.w;
        }
        if (NT) {
            __builtin_nontemporal_store(v.x, &c[i].x);
            __builtin_nontemporal_store(v.y, &c[i].y);
            __builtin_nontemporal_store(v.z, &c[i].z);
            __builtin_nontemporal_store(v.w, &c[i].w);
        } else {
            c[i] = v;
        }
    }
}

hipError_t launch_probe(float* c, const float* a, const float* b, int64_t n, int kind, bool nontemporal,
                        int blocks, hipStream_t s) {
    const int64_t n4 = n / 4;
    float4* c4 = reinterpret_cast<float4*>(c);
    const float4* a4 = reinterpret_cast<const float4*>(a);
    const float4* b4 = reinterpret_cast<const float4*>(b);
    if (kind == 0 && !nontemporal) hipLaunchKernelGGL((k_probe<0, false>), dim3(blocks), dim3(256), 0, s, c4, a4, b4, n4);
    if (kind == 0 && nontemporal) hipLaunchKernelGGL((k_probe<0, true>), dim3(blocks), dim3(256), 0, s, c4, a4, b4, n4);
    if (kind == 1 && !nontemporal) hipLaunchKernelGGL((k_probe<1, false>), dim3(blocks), dim3(256), 0, s, c4, a4, b4, n4);
    if (kind == 1 && nontemporal) hipLaunchKernelGGL((k_probe<1, true>), dim3(blocks), dim3(256), 0, s, c4, a4, b4, n4);
    return hipGetLastError();
}

}  // namespace jac
