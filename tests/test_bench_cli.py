"""bench.py's command line on the host: it measures one GPU only, so any
--gpus other than 1 ends with exit status 2 and a message, before anything
touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""
