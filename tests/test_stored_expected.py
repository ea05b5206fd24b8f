"""The stored expected values (tests/golden/expected_*.json, written by
tests/golden/make_expected.py from the oracle alone) against what the pages
state, on the CPU.

Block-asynchronous acceptance (page "stencil-jacobian.vercel.app", section 02,
kernel (c)): at the benchmark size N = 8192, r = 10, the oracle's block-async
solves reach rho < 1e-5 at every step and their fields stay within
1e-4 * ||b_A|| of the exact method's, step by step; the generator measured
that margin with the oracle's synchronous solve beside it.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, f"expected_{name}.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["C3_async_D8_32x16", "C3_async_D4_32x8"])
def test_async_within_page_tolerance_of_exact_solution(name):
    exp = load(name)
    sync = load("C3")
    assert exp["N"] == sync["N"] == 8192 and exp["r"] == sync["r"] == 10.0
    assert exp["sync_sweeps"] == sync["sweeps"]  # the same exact solve as the stored one
    rho = [np.uint32(int(h, 16)).view(np.float32) for h in exp["rho_bits"]]
    assert all(q < np.float32(1e-5) for q in rho)
    margins = exp["max_diff_over_bA"]
    assert len(margins) == exp["steps"] == 10
    assert all(0.0 < m <= 1e-4 for m in margins), margins
    # the staleness error accumulates over the steps (each step's solve leaves
    # a difference of up to about rho * ||b_A|| behind)
    assert margins[-1] == max(margins)
    # more sweeps than the exact method, by the extra-sweep ratio the page reports
    s = sum(exp["sweeps"]) / sum(sync["sweeps"])
    assert 1.0 < s < 2.0


@pytest.mark.parametrize("M", list(range(9, 17)))
def test_deep_interval_counts(M):
    """Temporal blocking with D > 8 checks every D sweeps (the oracle with
    M = D): each step's count is a multiple of M, at most one interval more
    than the M = 8 count rounded up, and every accepted rho is below tol."""
    exp = load(f"C3_M{M}")
    base = load("C3")
    assert exp["M"] == M
    for k, k8, h in zip(exp["sweeps"], base["sweeps"], exp["rho_bits"]):
        assert k % M == 0
        assert k8 - 8 < k <= k8 + M
        assert np.uint32(int(h, 16)).view(np.float32) < np.float32(1e-5)
