"""bench.py's command line, on the CPU: it measures one GPU only, so --gpus N with N > 1 ends at once with
exit status 2 and a message that says so (before anything touches a GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=60, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""  # no JSON line
