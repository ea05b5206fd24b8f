/* Exhaustive host check of the constant-divisor quotient used by the sweep:
 * q0 = RN(n*y), e = fma(-q0, d, n), q = fma(e, y, q0) with y = RN(1/d)
 * (Markstein, IBM J. Res. Dev. 34(1), 1990), compared with the correctly
 * rounded n / d of the host's IEEE division on every float n except Inf, NaN
 * and -0.  Prints the number of mismatches.  Needs a host with a hardware
 * fused multiply-add; build with -O3 -mfma -ffp-contract=off -fopenmp. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s d\n", argv[0]); return 2; }
    const float d = strtof(argv[1], NULL);
    const float y = 1.0f / d;
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t hi = 0; hi < (1 << 16); ++hi) {
        for (uint32_t lo = 0; lo < (1u << 16); ++lo) {
            const uint32_t bits = ((uint32_t)hi << 16) | lo;
            const int skip = (bits & 0x7F800000u) == 0x7F800000u || bits == 0x80000000u;
            const float n = from_bits(bits);
            const float q0 = n * y;
            const float e = fmaf(-q0, d, n);
            const float q = fmaf(e, y, q0);
            bad += (uint64_t)(!skip & (to_bits(q) != to_bits(n / d)));
        }
    }
    printf("%llu\n", (unsigned long long)bad);
    return 0;
}
