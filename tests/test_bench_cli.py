"""bench.py's command line on the CPU: a request for more than one GPU ends
at once with a message (the library has no multi-GPU mode), before any
device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps",
                        "1", "--warmup", "0"], capture_output=True, text=True, timeout=120,
                       cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU only" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or "{" not in r.stdout   # no JSON line
