"""bench.py's command-line contract, checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    """The measurement is of one GPU; asked for more, bench.py says so and
    exits non-zero before it touches a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""
