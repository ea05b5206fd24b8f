"""The C client of include/jacobi.h (tests/abi_client.c, built by
__graft_entry__.build()) on the GPU: a process that owns its workspace
(hipMalloc) and its stream, with no Python or PyTorch in it, solves the
point-source workload of page "stencil-jacobian.vercel.app", section 01
(N = 512, r = 1, three steps) and matches the oracle's stored result bit for
bit."""
import os
import subprocess

import numpy as np
import pytest

import jacobi_stencil_amd as jac
from jacobi_stencil_amd import build as libbuild
from tests.gpu_helpers import field_hash, load_expected, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kernel,D", [(jac.JAC_SYNC, 1), (jac.JAC_TBLOCK, 8), (jac.JAC_TBLOCK, 11)])
def test_c_client_matches_stored_oracle(kernel, D, tmp_path):
    exp = load_expected("C1")
    assert exp is not None and exp["source"] == "point"
    exe = libbuild.ABI_CLIENT
    assert os.path.exists(exe), "tests/abi_client is not built: run __graft_entry__.build()"
    N, r, steps = exp["N"], exp["r"], exp["steps"]
    out = tmp_path / "field.bin"
    say("abi_client", kernel, D)
    proc = subprocess.run([exe, str(N), repr(r), str(steps), str(kernel), str(D), str(out)],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stderr
    raw = out.read_bytes()
    sweeps = np.frombuffer(raw, "<i8", count=steps)
    rho = np.frombuffer(raw, "<f4", count=steps, offset=8 * steps)
    u = np.frombuffer(raw, "<f4", offset=12 * steps).reshape(N, N)
    assert sweeps.tolist() == exp["sweeps"]
    assert [f"{x:08x}" for x in rho.view(np.uint32)] == exp["rho_bits"]
    assert field_hash(u) == exp["field_sha256"][-1]
