#pragma once
// check_predict.h -- final-check prediction for the overlapped-check driver
// (host code only; the CPU tests compile it on its own).
//
// The check that ends a step is normally fused into a launch whose sweeps are then thrown away (a whole
// interval: eight launches of the synchronous sweep).  Once the last three
// checks of the step fall at a steady rate, rho of a later check is
// extrapolated geometrically; if it falls below margin * tol, that check is
// queued as a residual pass alone (8 bytes per point) with nothing behind it.
// If it does not converge after all, the interval it skipped is queued next
// from the same iterate.  The iterates, counts and rho are those of the
// unpredicted order; only which launches run changes.

#include <cmath>
#include <cstdint>

namespace jac {

constexpr float kPredictMargin = 0.97f;

// Temporal blocking through the launch driver: a check that is not expected
// to stop measures the residual on every kSampleRows-th row only.  That
// maximum bounds R from below, so a sample at or above tol shows that the
// step goes on, exactly as the full residual would; a sample below tol is
// checked again in full.  A check predicted below kSampleFar * tol, or within
// two intervals of the previous step's sweep count, measures every row.
constexpr int kSampleRows = 8;
constexpr float kSampleFar = 1.25f;

struct CheckHistory {
    float rho[3] = {0.0f, 0.0f, 0.0f};  // rho of the last three checks of the step, newest first
    int64_t last = 0;                   // the check rho[0] belongs to (0: none yet)
    int n = 0;
    void push(int64_t g, float r) {
        rho[2] = rho[1];
        rho[1] = rho[0];
        rho[0] = r;
        last = g;
        n = n < 3 ? n + 1 : 3;
    }
    // is check g (> last) predicted to converge?
    bool predicts_stop(int64_t g, float tol, float margin) const {
        if (margin <= 0.0f || n < 3 || g <= last) return false;
        if (!(rho[0] > 0.0f && rho[1] > 0.0f && rho[2] > 0.0f)) return false;  // also excludes NaN
        const double q1 = (double)rho[0] / rho[1], q0 = (double)rho[1] / rho[2];
        if (!(q1 < 1.0 && q0 < 1.0) || std::fabs(q1 / q0 - 1.0) > 0.02) return false;
        const double pred = (double)rho[0] * std::pow(q1, (double)(g - last));
        return pred < (double)margin * (double)tol;
    }
};

}  // namespace jac
