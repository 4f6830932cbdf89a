"""bench.py's command line on the CPU: a request for more than one GPU exits at once with
status 2 and a message (the bench measures one MI355X), before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in (2, 8):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                           text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, r
        assert "one GPU only" in r.stderr and r.stdout == ""
