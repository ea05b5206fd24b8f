"""The sweep divides by the constant d = 1 + 4r through RN(1/d) and one fma
correction, without a special-case fixup.  On the host, with IEEE division as
the reference, that quotient must be exact on every float numerator other than
Inf, NaN and -0 for the divisors of the measured workloads (r = 1, 10, 100),
and a plainly wrong variant must be caught.  The library repeats the check on
the device for its own d at create time."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _fma_host() -> bool:
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None or not _fma_host():
        pytest.skip("needs gcc and a host with hardware fma")
    exe = str(tmp_path_factory.mktemp("div") / "division_check")
    subprocess.run(["gcc", "-O3", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    os.path.join(HERE, "division_check.c"), "-o", exe, "-lm"], check=True)
    return exe


@pytest.mark.slow
@pytest.mark.parametrize("r", [1.0, 10.0, 100.0])
def test_constant_divisor_quotient_exhaustive(checker, r):
    d = np.float32(1.0) + np.float32(4.0) * np.float32(r)
    out = subprocess.run([checker, repr(float(d))], check=True, capture_output=True, text=True).stdout
    assert int(out) == 0


def test_quotient_without_correction_fails():
    """Negative control on a sample: RN(n * RN(1/d)) alone is not the quotient."""
    d = np.float32(41.0)
    y = np.float32(1.0) / d
    n = np.random.default_rng(0).uniform(1.0, 1000.0, 200000).astype(np.float32)
    assert np.count_nonzero((n * y) != (n / d)) > 1000
