"""Each plausible mistake planted in a copy of the oracle must fail one pin.

The mutants are built from oracle/jacobi_oracle.c by one textual replacement
each, compiled into a temporary directory, and the pin suite
(tests/test_oracle.py) is run against them in a subprocess.  This runs on the
CPU only and never touches the library path.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "jacobi_oracle.c")

MUTANTS = {
    "sum_order_north_first": ("float S = uE + uW;\n    S = S + uN;", "float S = uN + uE;\n    S = S + uW;"),
    "wrong_south_index": ("uS = U[c + P];", "uS = U[c + P + 1];"),
    "transposed_neighbours": ("float uE = U[c + 1], uW = U[c - 1], uN = U[c - P], uS = U[c + P];",
                              "float uE = U[c + P], uW = U[c - P], uN = U[c - 1], uS = U[c + 1];"),
    "residual_drops_south": ("    e = e + (U[c + P] - C);\n", ""),
    "residual_sign": ("return bc + t;", "return bc - t;"),
    "norm_without_boundary": ("float v = B[at(N, i, j)] + r * g;", "float v = B[at(N, i, j)];"),
    "diag_three_r": ("float four_r = 4.0f * r;", "float four_r = 3.0f * r;"),
    "check_on_previous_iterate": ("float R = residual_padded(N, r, cur, B);",
                                  "float R = residual_padded(N, r, nxt, B);"),
    "rhs_misses_source": ("= U[at(N, i, j)] + s[(size_t)i * N + j];", "= U[at(N, i, j)];"),
    "async_gauss_seidel_in_tile": ("nxt[l] = jacobi_point(cur, l, lp, bl[l], r, d);",
                                   "cur[l] = jacobi_point(cur, l, lp, bl[l], r, d); nxt[l] = cur[l];"),
    "async_halo_from_rhs": ("cur[(size_t)a * lp + c] = U[g];",
                            "cur[(size_t)a * lp + c] = (a == 0 || c == 0 || a == h + 1 || c == w + 1) ? B[g] : U[g];"),
    "overlap_one_sided": ("int ex0 = x0 - o < 0 ? 0 : x0 - o, ex1 = x1 + o > N ? N : x1 + o;",
                          "int ex0 = x0, ex1 = x1 + o > N ? N : x1 + o;"),
    "overlap_writes_widened_region": ("V[at(N, i, j)] = cur[(size_t)(i - ey0 + 1) * lp + (size_t)(j - ex0 + 1)];",
                                      "{ V[at(N, i, j)] = cur[(size_t)(i - ey0 + 1) * lp + (size_t)(j - ex0 + 1)];"
                                      " if (i == y0 && y0 > ey0) V[at(N, i - 1, j)] = cur[(size_t)(i - ey0) * lp + "
                                      "(size_t)(j - ex0 + 1)]; }"),
    "asc_not_latched": ("if (t > D) D = t;", "D = t;"),
    "desc_thresholds_shifted": ("if (q >= 1e-2f) return 8;", "if (q >= 1e-1f) return 8;"),
    "desc_levels_scaled_by_dmax": ("int t = cap_depth(desc_level(q), Dmax);",
                                   "int t = cap_depth(desc_level(q) * Dmax / 8 < 1 ? 1 : desc_level(q) * Dmax / 8, Dmax);"),
    "desc_starts_at_dmax": ("if (ctrl == ORC_G_DESC) D = cap_depth(8, Dmax);", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    msrc = tmp_path / "jacobi_oracle.c"
    msrc.write_text(src.replace(old, new))
    (tmp_path / "jacobi_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "jacobi_oracle.h")).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(msrc), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, JACOBI_ORACLE_LIB=str(lib))
    # under parallel test workers, share the cores out: OpenMP threads that
    # spin at barriers on oversubscribed cores slow the pins a hundredfold
    workers = int(os.environ.get("PYTEST_XDIST_WORKER_COUNT", "1"))
    if workers > 1:
        env["OMP_NUM_THREADS"] = str(max(1, (os.cpu_count() or 1) // workers))
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode == 1, f"mutant {name} passed every pin:\n{proc.stdout[-2000:]}"
