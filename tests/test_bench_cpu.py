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


def _bench_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_prefill_flops_counts_causal_pairs():
    """The chunk's FLOPs are 4 * 128 * heads per causal (query, key) pair:
    query i of a row's n queries sits at position L - n + i and sees that
    many keys plus itself.  Counted here by brute force over the pairs."""
    from types import SimpleNamespace

    bench = _bench_module()
    b = SimpleNamespace(rows=3, q_counts=[5, 1, 3], context_lens=[9, 40, 3], num_heads=7)
    pairs = 0
    for n, L in zip(b.q_counts, b.context_lens):
        if n < 2:
            continue  # a decode row is not prefill work
        pairs += sum(1 for i in range(n) for j in range(L) if j <= L - n + i)
    assert bench.prefill_flops(b) == 4.0 * 128 * 7 * pairs


def test_counter_summary_is_refused_when_its_sources_changed(tmp_path):
    """A committed counter summary feeds `traffic` only while the kernel
    sources hash to the value recorded in it."""
    import json

    bench = _bench_module()
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of a kernel\n")
    rec_path = tmp_path / "counters.json"
    rec_path.write_text(json.dumps({"source_sha256": bench.source_digest([str(src)]),
                                    "traffic_bytes_per_launch": 123.0}))
    assert bench.counted_record(str(rec_path), [str(src)])["traffic_bytes_per_launch"] == 123.0
    src.write_text("// another version\n")
    assert bench.counted_record(str(rec_path), [str(src)]) is None
    assert bench.counted_record(str(tmp_path / "missing.json"), [str(src)]) is None
