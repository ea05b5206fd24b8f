/*
 * abi_client.c -- a plain C11 program that uses libjacobi only through
 * include/jacobi.h, the way a C caller would: it owns the device workspace
 * (hipMalloc) and the HIP stream it hands to jac_create, and checks the
 * interface's ownership, ordering and error rules.
 *
 * The solve it runs is the one of page "stencil-jacobian.vercel.app",
 * section 01 "The problem": backward-Euler steps of the heat equation on an
 * N x N grid with a point source at the centre cell, each step iterated to
 * rho < 1e-5.
 *
 *   abi_client --cpu
 *       Calls that need no GPU: option defaults, workspace sizes, and the
 *       argument errors jac_create and the step calls report before they
 *       touch the device.  Exit status 0 when every check holds.
 *   abi_client N r steps kernel D out.bin
 *       hipMalloc's a workspace of jac_workspace_bytes(N) bytes, creates a
 *       stream, runs `steps` steps with kernel / D (the other options at their
 *       defaults), then writes to out.bin: int64 sweeps[steps], float
 *       rho[steps], float field[N*N] (row-major, little-endian).  The source
 *       is s = r at unknown (N/2, N/2) and 0 elsewhere (f = 1/h^2 at the centre
 *       cell with dt = r h^2).
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "jacobi.h"

/* The option block's layout, as the header declares it (checked at compile time). */
_Static_assert(sizeof(jac_opts) == 56, "jac_opts is 56 bytes");
_Static_assert(offsetof(jac_opts, kernel) == 0, "kernel");
_Static_assert(offsetof(jac_opts, driver) == 4, "driver");
_Static_assert(offsetof(jac_opts, D) == 8, "D");
_Static_assert(offsetof(jac_opts, tile_x) == 12, "tile_x");
_Static_assert(offsetof(jac_opts, tile_y) == 16, "tile_y");
_Static_assert(offsetof(jac_opts, M) == 20, "M");
_Static_assert(offsetof(jac_opts, tol) == 24, "tol");
_Static_assert(offsetof(jac_opts, band_rows) == 28, "band_rows");
_Static_assert(offsetof(jac_opts, max_sweeps) == 32, "max_sweeps");
_Static_assert(offsetof(jac_opts, checks) == 40, "checks");
_Static_assert(offsetof(jac_opts, controller) == 44, "controller");
_Static_assert(offsetof(jac_opts, overlap) == 48, "overlap");
_Static_assert(offsetof(jac_opts, reserved) == 52, "reserved");

static int failures = 0;

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "abi_client: check failed at line %d: %s (%s)\n",    \
                    __LINE__, #cond, jac_last_error());                          \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static int cpu_checks(void) {
    jac_opts o;
    memset(&o, 0xAB, sizeof o);
    jac_opts_default(&o);
    CHECK(o.kernel == JAC_SYNC && o.driver == JAC_LAUNCH && o.D == 1);
    CHECK(o.tile_x == 32 && o.tile_y == 8 && o.M == 8 && o.tol == 1e-5f);
    CHECK(o.band_rows == 0 && o.max_sweeps == 1000000 && o.checks == JAC_CHECKS_OVERLAPPED);
    CHECK(o.controller == JAC_STATIC && o.overlap == 0 && o.reserved == 0);

    CHECK(jac_workspace_bytes(0) == 0 && jac_workspace_bytes(65537) == 0);
    const size_t w512 = jac_workspace_bytes(512);
    CHECK(w512 >= (size_t)4 * 512 * 512 * sizeof(float) && w512 % 256 == 0);
    CHECK(jac_workspace_bytes(1024) > w512);

    /* argument errors come back as status codes, with a message, before any
     * device work; *out is cleared */
    jac_t ctx = (jac_t)(uintptr_t)0x1;
    void* fake = (void*)(uintptr_t)4096; /* aligned, never dereferenced on these paths */
    CHECK(jac_create(0, 1.0f, NULL, fake, w512, NULL, &ctx) == JAC_EINVAL && ctx == NULL);
    CHECK(strlen(jac_last_error()) > 0);
    CHECK(jac_create(512, -1.0f, NULL, fake, w512, NULL, &ctx) == JAC_EINVAL);
    CHECK(jac_create(512, 1.0f, NULL, NULL, w512, NULL, &ctx) == JAC_EINVAL);
    CHECK(jac_create(512, 1.0f, NULL, (char*)fake + 4, w512, NULL, &ctx) == JAC_EINVAL);
    CHECK(jac_create(512, 1.0f, NULL, fake, w512 - 256, NULL, &ctx) == JAC_ENOMEM);
    CHECK(jac_create(512, 1.0f, NULL, fake, w512, NULL, NULL) == JAC_EINVAL);
    int64_t k = 0;
    float rho = 0.0f;
    CHECK(jac_step(NULL, &o, &k, &rho) == JAC_EINVAL);
    CHECK(jac_solve(NULL, 10, &o, NULL, NULL) == JAC_EINVAL);
    CHECK(jac_sweep(NULL, &o, 8, NULL) == JAC_EINVAL);
    CHECK(jac_get_field(NULL, NULL) == JAC_EINVAL);
    CHECK(jac_destroy(NULL) == JAC_OK);
    return failures == 0 ? 0 : 1;
}

#define HIPCHECK(call)                                                                 \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "abi_client: %s: %s\n", #call, hipGetErrorString(e_));    \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

static int gpu_run(int N, float r, int steps, int kernel, int D, const char* path) {
    const size_t n = (size_t)N * N;
    float* src = (float*)calloc(n, sizeof(float));
    float* field = (float*)malloc(n * sizeof(float));
    int64_t* sweeps = (int64_t*)calloc((size_t)steps, sizeof(int64_t));
    float* rho = (float*)calloc((size_t)steps, sizeof(float));
    if (!src || !field || !sweeps || !rho) return 2;
    src[(size_t)(N / 2) * N + (size_t)(N / 2)] = r;

    const size_t ws = jac_workspace_bytes(N);
    void* work = NULL;
    HIPCHECK(hipMalloc(&work, ws)); /* hipMalloc returns at least 256-byte alignment */
    hipStream_t stream = NULL;
    HIPCHECK(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));

    jac_t ctx = NULL;
    CHECK(jac_create(N, r, src, work, ws, stream, &ctx) == JAC_OK && ctx != NULL);
    /* the source is copied during jac_create: changing the caller's array
     * afterwards must not change the solve */
    src[(size_t)(N / 2) * N + (size_t)(N / 2)] = 1e30f;

    jac_opts o;
    jac_opts_default(&o);
    o.kernel = kernel;
    o.D = D;
    CHECK(jac_solve(ctx, steps, &o, sweeps, rho) == JAC_OK);
    /* a bad option is refused without touching the field */
    jac_opts bad = o;
    bad.M = 0;
    CHECK(jac_step(ctx, &bad, NULL, NULL) == JAC_EINVAL);
    CHECK(jac_get_field(ctx, field) == JAC_OK);
    /* after a blocking read-back the context's stream holds no more work */
    CHECK(hipStreamQuery(stream) == hipSuccess);
    CHECK(jac_destroy(ctx) == JAC_OK);
    /* the workspace and the stream stay the caller's: both still usable */
    HIPCHECK(hipMemsetAsync(work, 0, 256, stream));
    HIPCHECK(hipStreamSynchronize(stream));
    HIPCHECK(hipStreamDestroy(stream));
    HIPCHECK(hipFree(work));

    FILE* f = fopen(path, "wb");
    if (!f) return 2;
    int ok = fwrite(sweeps, sizeof(int64_t), (size_t)steps, f) == (size_t)steps &&
             fwrite(rho, sizeof(float), (size_t)steps, f) == (size_t)steps &&
             fwrite(field, sizeof(float), n, f) == n;
    ok = (fclose(f) == 0) && ok;
    free(src);
    free(field);
    free(sweeps);
    free(rho);
    if (!ok) return 2;
    return failures == 0 ? 0 : 1;
}

int main(int argc, char** argv) {
    if (argc == 2 && strcmp(argv[1], "--cpu") == 0) return cpu_checks();
    if (argc == 7) {
        const int N = atoi(argv[1]);
        const float r = (float)atof(argv[2]);
        const int steps = atoi(argv[3]);
        const int kernel = atoi(argv[4]);
        const int D = atoi(argv[5]);
        if (N < 1 || steps < 1) return 2;
        return gpu_run(N, r, steps, kernel, D, argv[6]);
    }
    fprintf(stderr, "usage: %s --cpu | N r steps kernel D out.bin\n", argv[0]);
    return 2;
}
