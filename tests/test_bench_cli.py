"""bench.py's command line on a machine without a GPU: the multi-GPU request
is refused (one GPU per run; no figure at several GPUs) before anything
touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr
    assert res.stdout.strip() == ""          # no JSON line
