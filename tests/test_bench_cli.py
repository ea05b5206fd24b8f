"""bench.py measures one GPU: asking for more exits with a message, before any
device work (CPU only)."""
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
