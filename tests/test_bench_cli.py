"""bench.py's command-line contract on a host without a GPU: more than one GPU
is refused with a message before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                           capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert r.returncode == 2, (n, r.returncode, r.stderr[-500:])
        assert "one GPU" in r.stderr and r.stdout == ""
