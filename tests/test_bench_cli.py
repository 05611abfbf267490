"""bench.py's command line on the CPU: the one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one gpu" in r.stderr.lower(), r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration it does not run
