// kernels_copy.hip -- the N x N field between the padded planes and a
// contiguous row-major block, for the host transfers at the C interface
// (jac_create's source, jac_get_field, jac_set_field).  The host side moves
// one contiguous block with a plain 1-D copy; this kernel changes the pitch
// on the device.
#include "jacobi_internal.h"

namespace jac {

// dst[i * dpitch + j] = src[i * spitch + j] for 0 <= i, j < N (offsets of
// element (0, 0) already applied to both pointers)
__global__ __launch_bounds__(256) void k_copy_rect(float* __restrict__ dst, int64_t dpitch,
                                                   const float* __restrict__ src, int64_t spitch, int N) {
    for (int64_t i = blockIdx.y; i < N; i += gridDim.y) {
        const float* s = src + i * spitch;
        float* d = dst + i * dpitch;
        for (int j = blockIdx.x * 256 + (int)threadIdx.x; j < N; j += (int)gridDim.x * 256) d[j] = s[j];
    }
}

hipError_t launch_copy_rect(float* dst, int64_t dpitch, const float* src, int64_t spitch, int N, hipStream_t s) {
    if (N < 1) return hipSuccess;
    const int gx = (N + 255) / 256 < 32 ? (N + 255) / 256 : 32;
    const int gy = N < 4096 ? N : 4096;
    hipLaunchKernelGGL(k_copy_rect, dim3(gx, gy), dim3(256), 0, s, dst, dpitch, src, spitch, N);
    return hipGetLastError();
}

}  // namespace jac
