"""The final-check prediction rule of the overlapped driver (host code,
`jacobi_stencil_amd/csrc/check_predict.h`), compiled on the CPU with g++: it
fires only on a history of three checks falling at a steady rate, and only
when the geometric extrapolation lands below margin * tol.  Results never
depend on it (the GPU tests hold that); this pins the rule itself."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "jacobi_stencil_amd", "csrc")

DRIVER = r'''
#include "check_predict.h"
#include <cstdio>
#include <cmath>
using jac::CheckHistory;
static CheckHistory hist3(float a, float b, float c) {  // oldest first
    CheckHistory h; h.push(1, a); h.push(2, b); h.push(3, c); return h;
}
int main() {
    const float tol = 1e-5f, m = 0.97f;
    CheckHistory empty;
    CheckHistory two; two.push(1, 2e-5f); two.push(2, 1.6e-5f);
    // rho 6.25e-5, 5e-5, 4e-5: ratio 0.8; check 3 + k extrapolates to 4e-5 * 0.8^k
    const CheckHistory steady = hist3(6.25e-5f, 5e-5f, 4e-5f);
    std::printf("empty %d\n", empty.predicts_stop(1, tol, m));
    std::printf("two %d\n", two.predicts_stop(4, tol, m));
    std::printf("steady+1 %d\n", steady.predicts_stop(4, tol, m));
    std::printf("steady+6 %d\n", steady.predicts_stop(9, tol, m));   // 1.05e-5
    std::printf("steady+7 %d\n", steady.predicts_stop(10, tol, m));  // 8.4e-6
    std::printf("steady_past %d\n", steady.predicts_stop(3, tol, m));
    std::printf("margin0 %d\n", steady.predicts_stop(10, tol, 0.0f));
    std::printf("huge+1 %d\n", steady.predicts_stop(4, tol, 1e30f));
    std::printf("unsteady %d\n", hist3(1.6e-4f, 8e-5f, 4e-5f * 0.8f * 2.0f).predicts_stop(10, tol, m));
    std::printf("ratios_3pct %d\n", hist3(6.25e-5f, 5e-5f, 5e-5f * 0.824f).predicts_stop(20, tol, m));
    std::printf("ratios_1pct %d\n", hist3(6.25e-5f, 5e-5f, 5e-5f * 0.808f).predicts_stop(20, tol, m));
    std::printf("rising %d\n", hist3(4e-5f, 5e-5f, 6.25e-5f).predicts_stop(20, tol, 1e30f));
    std::printf("nan %d\n", hist3(6.25e-5f, NAN, 4e-5f).predicts_stop(20, tol, 1e30f));
    std::printf("zero %d\n", hist3(6.25e-5f, 5e-5f, 0.0f).predicts_stop(20, tol, 1e30f));
    CheckHistory slid = steady; slid.push(4, 3.2e-5f);  // the newest three: ratio still 0.8
    std::printf("slid+6 %d\n", slid.predicts_stop(10, tol, m));   // 3.2e-5 * 0.8^6 = 8.4e-6
    std::printf("slid_n %d\n", slid.n);
    return 0;
}
'''


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    d = tmp_path_factory.mktemp("predict")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    exe = d / "driver"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return dict(line.split() for line in out.strip().splitlines())


@pytest.mark.parametrize("case,want", [
    ("empty", "0"), ("two", "0"),                       # fewer than three checks
    ("steady+1", "0"), ("steady+6", "0"), ("steady+7", "1"),  # the threshold margin * tol
    ("steady_past", "0"), ("margin0", "0"), ("huge+1", "1"),
    ("unsteady", "0"), ("ratios_3pct", "0"), ("ratios_1pct", "1"),  # ratios must agree within 2 %
    ("rising", "0"), ("nan", "0"), ("zero", "0"),
    ("slid+6", "1"), ("slid_n", "3"),
])
def test_prediction_rule(results, case, want):
    assert results[case] == want, case
