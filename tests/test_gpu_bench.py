"""Benchmark smoke test on the GPU: bench.py runs every leg at small settings in
a child process and prints one JSON line with the fields the measurement
contract asks for (metric, value, roofline, and each leg's record)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_bench_runs_every_leg():
    pytest.importorskip("torch").cuda.is_available() or pytest.skip("no GPU")
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--cpu-seconds", "3",
           "--trace-steps", "12"]
    print("bench smoke:", " ".join(cmd[1:]), flush=True)
    # the child's progress lines go straight to this process's stderr
    res = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900, cwd=ROOT)
    assert res.returncode == 0, f"bench.py exited with {res.returncode}"
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("{")][-1]
    rec = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "dtype", "data", "config", "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["value"] > 0 and rec["config"]["workload"]
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and 0 < roof["frac"] < 1 and roof["achievable"]["slab_read_gb_s"] > 0
    for leg in ("prefill", "trace", "long_context", "gqa_decode", "gqa8_decode", "fp8_decode", "block_copy", "tiny_decode"):
        assert rec[leg], leg
    assert 0 < rec["prefill"]["roofline"]["frac"] < 1
    assert 0 < rec["prefill"]["roofline"]["frac_of_achievable"] < 1
    assert rec["trace"]["steps"] == 12 and rec["trace"]["pool_drained"]
    assert rec["parity_step0"]["pass"], rec["parity_step0"]
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    print(f"bench smoke ok: {rec['value']:.3g} KV-tokens/s, roofline frac {roof['frac']:.3f}", flush=True)
