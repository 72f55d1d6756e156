"""bench.py's command line on the CPU: a request for several GPUs is refused
with a message and exit status 2 (the path runs its N virtual ranks on one
GPU), before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr or "single MI355X" in res.stderr
    assert res.stdout.strip() == ""
