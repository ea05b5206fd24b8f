"""bench.py on the CPU: asking for more than one GPU exits with a message before
any device work, and the counter-file summary picks the right launches."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout.strip() == ""


def test_counters_summary_takes_the_most_called_kernel_and_skips_no_op_launches(tmp_path, capsys):
    import csv
    import json

    sys.path.insert(0, ROOT)
    import bench

    main_k = "void jac::k_tblock<8, true, true>(float const*, float const*, float*, jac::StepArgs, int)"
    first_k = "void jac::k_tblock<8, false, true>(float const*, float const*, float*, jac::StepArgs, int)"
    rows = []
    # (kernel, dispatch, start, end, {counter: value}); dispatch 3 returned at once after a stop
    for k, d, t0, t1, vals in ((main_k, 1, 0, 200_000, {"A": 10.0, "B": 1.0}),
                               (main_k, 2, 300_000, 490_000, {"A": 20.0, "B": 3.0}),
                               (main_k, 3, 500_000, 501_000, {"A": 0.0, "B": 0.0}),
                               (first_k, 4, 600_000, 900_000, {"A": 99.0, "B": 99.0}),
                               ("jac::k_reduce(long, int, jac::StepArgs)", 5, 0, 4000, {"A": 7.0})):
        for name, v in vals.items():
            rows.append({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": name, "Counter_Value": v,
                         "Start_Timestamp": t0, "End_Timestamp": t1})
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    bench.counters_from([str(path)], "tblock")
    res = json.loads(capsys.readouterr().out)
    assert res["kernel"] == main_k and res["launches"] == 2
    assert res["median"] == {"A": 15.0, "B": 2.0}


def test_cpu_only_times_the_oracle_without_a_device():
    import json

    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "C5", "--cpu-only",
                           "--cpu-threads", "1", "--cpu-steps", "2"], capture_output=True, text=True, timeout=300,
                          cwd=ROOT)
    assert proc.returncode == 0, proc.stderr
    res = json.loads(proc.stdout.strip().splitlines()[-1])
    cb = res["cpu_baseline"]
    assert res["config"] == "C5" and cb["kind"] == "oracle" and cb["cores"] == 1
    assert cb["value"] > 0 and "(488 sweeps" in cb["sample"]  # two steps of C5 at r = 10: 248 + 240
    assert cb["host"]["nproc"] >= 1
