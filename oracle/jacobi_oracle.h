/*
 * jacobi_oracle.h -- entry points of the plain CPU reference (test
 * infrastructure only; see jacobi_oracle.c for what each computes and which
 * passage of the pages it follows).  Arrays are N x N row-major float32
 * unknowns; the ghost ring (top 100, other sides 0) is built inside.
 */
#ifndef JACOBI_ORACLE_H
#define JACOBI_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2, ORC_ENOCONV = -4, ORC_ENAN = -5 };
enum { ORC_SYNC = 0, ORC_ASYNC = 2, ORC_WRONG_B = 3 };
enum { ORC_STATIC = 0, ORC_G_ASC = 1, ORC_G_DESC = 2, ORC_SCHED = 3 };

void  orc_set_threads(int n);
int   orc_get_threads(void);
float orc_diag(float r);
void  orc_rhs(int N, const float* u, const float* s, float* b);
float orc_rhs_norm(int N, float r, const float* b);
void  orc_sweep(int N, float r, const float* u, const float* b, float* out);
float orc_residual(int N, float r, const float* u, const float* b);
void  orc_async_launch(int N, float r, const float* u, const float* b, float* out, int tx, int ty, int D,
                       int o);
int   orc_solve(int N, float r, const float* s, float* u_io, int steps, float tol, int M, int mode,
                int D, int tx, int ty, int64_t max_sweeps, int64_t* sweeps, float* rho,
                float* R_log, int64_t log_cap, int64_t* log_n);
int   orc_solve_ex(int N, float r, const float* s, float* u_io, int steps, float tol, int M, int mode,
                   int Dmax, int tx, int ty, int o, int ctrl, const int* sched, int64_t sched_n,
                   int64_t max_sweeps, int64_t* sweeps, float* rho,
                   float* R_log, int* d_log, int64_t log_cap, int64_t* log_n);

#ifdef __cplusplus
}
#endif
#endif
