"""bench.py's command line on the CPU: more than one GPU is refused with a
JSON message and exit status 2, before any device is touched."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus_requested"] == 2 and "one GPU" in line["error"]
