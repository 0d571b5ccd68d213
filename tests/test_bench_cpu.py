"""bench.py's command-line contract that needs no GPU: one GPU only, so any
other --gpus value ends with a message and exit status 2 before torch or
the library is loaded."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    for n in (2, 8):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                           capture_output=True, text=True, timeout=60, cwd=ROOT)
        assert p.returncode == 2
        assert "one GPU only" in p.stderr and f"--gpus {n}" in p.stderr
        assert p.stdout == ""  # no JSON line
