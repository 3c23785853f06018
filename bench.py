#!/usr/bin/env python3
"""Benchmark: one decode step of the average-mix batch over all 32 layers.

A step is the whole hot path for one batch of 32 decode rows:
  host  grow block tables through the C++ block pool where a row crosses a
        16-token boundary, upload tables / lengths / positions (pinned, async);
  GPU   for each of 32 layers: KV append of the 32 new tokens, then paged
        decode attention (split-K kernel + merge kernel).
Rows advance one token per step, as in a real decode loop.

Workload: 32 rows, context = lognormal prompt (mean 1,250, clipped to
[50, 8000]) + U{1..300} generated tokens; KV pool of 7,152 blocks x
[32 layers, 2, 32 heads, 16, 128] FP16 (60 GB), blocks handed out from a
shuffled free list, values N(0,1).  Inputs are resident in HBM before the
timed region starts.

Prints one JSON line.  `value` is KV-tokens/s where one KV-token is a cached
token read across all 32 layers (524,288 bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-tokens/s + HBM TB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
LAYER_TOKEN_BYTES = 2 * 32 * 128 * 2          # K+V of one token, one layer
STEP_TOKEN_BYTES = LAYER_TOKEN_BYTES * 32       # all 32 layers


CSRC = os.path.join(ROOT, "paged_kv_cache_pkv_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "decode_average_mix_hbm_counters.json")
DECODE_SOURCES = [os.path.join(CSRC, n) for n in ("decode.hip", "decode_core.h", "device_common.h")]
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_chunk512_hbm_counters.json")
PREFILL_SOURCES = [os.path.join(CSRC, n) for n in ("prefill.hip", "decode_core.h", "device_common.h")]
APPEND_COUNTERS = os.path.join(ROOT, "profiles", "append_bulk_hbm_counters.json")
APPEND_SOURCES = [os.path.join(CSRC, n) for n in ("append.hip", "device_common.h")]
FP8_GQA_COUNTERS = os.path.join(ROOT, "profiles", "fp8_gqa_decode_average_mix_hbm_counters.json")
FP8_SOURCES = [os.path.join(CSRC, n) for n in ("fp8.hip", "decode_core.h", "device_common.h")]


def source_digest(sources=None) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in sources or DECODE_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counted_record(path, sources):
    """A committed rocprofv3 counter summary (JSON), or None when it is missing
    or the kernel sources have changed since the counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(sources):
        return None
    return rec


def fp8_gqa_traffic(kind):
    """HBM bytes per 8-bit ("fp8") or grouped-query ("gqa": groups of 4, "gqa8":
    groups of 8) decode call from the committed counter summary, or None when
    its sources have changed."""
    try:
        with open(FP8_GQA_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get(f"source_sha256_{kind}") != source_digest(FP8_SOURCES if kind == "fp8" else DECODE_SOURCES):
        return None
    return rec.get(f"{kind}_traffic_bytes_per_launch")


def counted_traffic():
    """HBM bytes per decode launch from the committed counter summary, or None."""
    rec = counted_record(COUNTERS, DECODE_SOURCES)
    return rec.get("traffic_bytes_per_launch") if rec else None


MFMA_F16_PEAK_TFLOPS = 2500.0


def prefill_flops(batch) -> float:
    """Causal (query, key) pairs of the rows with at least two queries x 4 x D x H."""
    total = 0
    for r in range(batch.rows):
        n = int(batch.q_counts[r])
        L = int(batch.context_lens[r])
        if n >= 2:
            total += n * (L - n + 1) + n * (n - 1) // 2  # sum over i < n of (L - n + i + 1)
    return 4.0 * 128 * batch.num_heads * total


def measure_prefill(torch, pkv, dev, stream, reps=20):
    """Chunked prefill on MFMA: a 512-token chunk at offset 7,488 of an 8,000-token
    prompt, alone and mixed with 31 average-mix decode rows in one launch,
    over a one-layer 7,152-block pool.  Returns a dict for the JSON line."""
    from workloads import SCALE, build_batch, c5_mixed, fill_normal_fp16_device

    pool = torch.empty((7152, 1, 2, 32, 16, 128), dtype=torch.int16, device=dev)
    fill_normal_fp16_device(pool, seed=2004)
    cache = pkv.PagedCache(pool)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    def timed(batch):
        tables, qs, lens = d(batch.block_tables), d(batch.query_start), d(batch.context_lens)
        q, k, v = d(batch.q[0]), d(batch.k_new[0]), d(batch.v_new[0])
        pos, rot = d(batch.positions), d(batch.request_of_token)
        T, maxq, maxL = batch.total_q, int(batch.q_counts.max()), int(batch.context_lens.max())
        ws = torch.empty(pkv.prefill_workspace_size(cache, batch.rows, T, maxq, maxL), dtype=torch.uint8, device=dev)
        out = torch.empty((T, 32, 128), dtype=torch.float16, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        pkv.append(cache, 0, k, v, pos, rot, tables, stream=stream)
        pkv.chunked_prefill_attention(cache, 0, out, q, qs, tables, lens, maxq, maxL, SCALE, ws, stream=stream)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            pkv.append(cache, 0, k, v, pos, rot, tables, stream=stream)
        ev[1].record(stream)
        for _ in range(reps):
            pkv.chunked_prefill_attention(cache, 0, out, q, qs, tables, lens, maxq, maxL, SCALE, ws, stream=stream)
        ev[2].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps, ev[1].elapsed_time(ev[2]) / reps

    def cold_prefill(batch, reps=10):
        """One prefill call with the 256 MB last-level cache scrubbed before
        every launch (a 512 MB streaming write, outside the timed launch)."""
        tables, qs, lens, q = d(batch.block_tables), d(batch.query_start), d(batch.context_lens), d(batch.q[0])
        T, maxq, maxL = batch.total_q, int(batch.q_counts.max()), int(batch.context_lens.max())
        ws = torch.empty(pkv.prefill_workspace_size(cache, batch.rows, T, maxq, maxL), dtype=torch.uint8, device=dev)
        out = torch.empty((T, 32, 128), dtype=torch.float16, device=dev)
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ms = []
        for _ in range(reps):
            scrub.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.chunked_prefill_attention(cache, 0, out, q, qs, tables, lens, maxq, maxL, SCALE, ws, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        del scrub
        return float(np.median(ms))

    def bulk_append(tokens, reps=20):
        """Append a whole prompt's K/V (one row, positions 0..tokens-1)."""
        b = build_batch(f"append{tokens}", 11, [tokens], [tokens], num_blocks=7152, with_pool=False)
        tables, pos, rot = d(b.block_tables), d(b.positions), d(b.request_of_token)
        k, v = d(b.k_new[0]), d(b.v_new[0])
        pkv.append(cache, 0, k, v, pos, rot, tables, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pkv.append(cache, 0, k, v, pos, rot, tables, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = tokens * 2 * LAYER_TOKEN_BYTES / (ms / 1e3) / 1e9  # each K/V byte read once, written once
        rec = counted_record(APPEND_COUNTERS, APPEND_SOURCES)
        traffic = rec.get("traffic_bytes_per_launch_by_tokens", {}).get(str(tokens)) if rec else None
        return {"tokens": tokens, "us": ms * 1e3, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}

    mixed = c5_mixed(with_pool=False)
    chunk = build_batch("chunk-only", 4, [8000], [512], num_blocks=7152, with_pool=False, stride=520)
    app_mixed_ms, mixed_ms = timed(mixed)
    _, chunk_ms = timed(chunk)
    chunk_cold_ms = cold_prefill(chunk)
    mixed_cold_ms = cold_prefill(mixed)
    appends = [bulk_append(n) for n in (512, 8000)]
    flops = prefill_flops(chunk)
    kv_mixed = float(mixed.context_lens.sum()) * LAYER_TOKEN_BYTES
    tflops = flops / (chunk_ms / 1e3) / 1e12
    rec = counted_record(PREFILL_COUNTERS, PREFILL_SOURCES)
    prefill_traffic = rec.get("traffic_bytes_per_launch") if rec else None
    ceiling = measure_mfma_ceiling(torch, stream)
    return {
        "workload": "512-token causal chunk at offset 7488 of an 8000-token prompt + 31 average-mix decode rows, "
                    "one layer, 32 heads x 128, FP16",
        "mixed_launch_us": mixed_ms * 1e3,
        "mixed_launch_cold_cache_us": mixed_cold_ms * 1e3,
        "mixed_kv_bytes": kv_mixed,
        "mixed_hbm_gb_s": kv_mixed / (mixed_ms / 1e3) / 1e9,
        "chunk_only_launch_us": chunk_ms * 1e3,
        "chunk_flops": flops,
        "chunk_only_cold_cache_us": chunk_cold_ms * 1e3,
        "append_543_tokens_us": app_mixed_ms * 1e3,
        "append_bulk_roofline": appends,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": prefill_traffic,
                     "kernel": "pkv_chunked_prefill_attention on the chunk alone (tile + merge launches)",
                     "achievable": ceiling,
                     "frac_of_achievable": tflops / ceiling["mfma_f16_tflops"] if ceiling else None},
    }


TRACE_SAMPLED = (10, 150, 299)  # timed-step indices whose outputs the oracle leg checks
TRACE_CHECK_ROWS = range(0, 64, 4)  # 16 of the 64 rows of each sampled step


def _run_trace(torch, steps, warm, shared_decode, cold_steps=20, checker=False):
    from paged_kv_cache_pkv_amd.trace import ContinuousBatchTrace

    tr = ContinuousBatchTrace(torch, seed=3, num_blocks=36864, max_rows=64, prefix_tokens=2000,
                              prompt_range=(50, 8000), answer_range=(1, 1000), shared_decode=shared_decode)
    chk = None
    if checker:
        from tests.trace_check import TraceChecker  # test infrastructure for the oracle leg

        chk = TraceChecker(tr)
    for _ in range(warm):
        snap = tr.step()
        if chk:
            chk.record(snap)
    torch.cuda.synchronize()
    rec = []
    for i in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        snap = tr.step(events=ev)
        if chk:
            chk.record(snap)
            if i in TRACE_SAMPLED:
                chk.keep(snap)
        sharers = sum(1 for r in tr.rows if r.shared)
        rec.append((ev, int(snap["lens"].sum()), sharers, snap["host_ms"], snap["stage_wait_ms"]))
    torch.cuda.synchronize()
    # cold: the 256 MB last-level cache scrubbed (a 512 MB write, not timed)
    # before each step's decode part
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=tr.dev)
    cold = []
    for _ in range(cold_steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        snap = tr.step(events=ev, before_decode=lambda: scrub.fill_(1))
        if chk:
            chk.record(snap)
        cold.append(ev)
    torch.cuda.synchronize()
    del scrub
    cold_ms = np.array([e[2].elapsed_time(e[3]) for e in cold])
    fill_ms = np.array([e[0].elapsed_time(e[1]) for e, _, _, _, _ in rec])
    step_ms = np.array([e[2].elapsed_time(e[3]) for e, _, _, _, _ in rec])
    with_host_ms = np.array([e[1].elapsed_time(e[3]) for e, _, _, _, _ in rec])
    host_ms = np.array([h for _, _, _, h, _ in rec])
    wait_ms = np.array([w for _, _, _, _, w in rec])
    tokens = np.array([t for _, t, _, _, _ in rec], dtype=np.float64)
    sharers = np.array([n for _, _, n, _, _ in rec], dtype=np.float64)
    joins = sum(1 for j in tr.log["joins"] if warm <= j[4] < warm + steps)
    prefix = tr.prefix_tokens
    tr.drain()
    assert tr.pool.num_free == 36864, "trace leaked blocks"
    del tr.pool_d
    return dict(step_ms=step_ms, fill_ms=fill_ms, tokens=tokens, sharers=sharers, joins=joins, prefix=prefix,
                with_host_ms=with_host_ms, host_ms=host_ms, wait_ms=wait_ms, cold_ms=cold_ms, checker=chk)


def measure_trace(torch, steps=300, warm=5, checkers=None):
    """Continuous-batching trace: up to 64 rows over a 36,864-block one-layer
    pool, prompts U{50..8000}, answers U{1..1000}, a 2,000-token prefix
    shared by reference counts; rows leave and are refilled every step.
    The decode part of a step (append one token per row, decode) is timed
    with events around its launches, separately from the fill of joining
    rows; the host's preparation before the launches (one batched table
    growth, the pinned upload of tables and lengths) is timed on the host and
    reported beside it, as is the step with it.  After the timed steps, 20
    more steps run with the last-level cache scrubbed before each decode part
    (cold).  The same seeded trace runs twice: with plain decode, and with the
    shared-prefix decode that reads the prefix once per step for every 32 rows
    holding it.  With `checkers` (a list), the outputs of three sampled steps
    are kept for the oracle leg."""
    want = checkers is not None
    p = _run_trace(torch, steps, warm, False, checker=want)
    s = _run_trace(torch, steps, warm, True, checker=want)
    if want:
        checkers.extend([("appending", p["checker"]), ("shared_prefix", s["checker"])])
    tokens, sharers, prefix = p["tokens"], p["sharers"], p["prefix"]
    assert np.array_equal(tokens, s["tokens"]) and np.array_equal(sharers, s["sharers"]), "the two traces diverged"
    # tokens the shared-prefix decode reads: the prefix once per tile of up to 32 sharing rows
    physical = tokens - prefix * (sharers - np.ceil(sharers / 32.0))

    def leg(d, extra):
        ms = d["step_ms"]
        out = {
            "decode_step_ms_p50": float(np.percentile(ms, 50)),
            "decode_step_ms_p90": float(np.percentile(ms, 90)),
            "decode_step_ms_max": float(ms.max()),
            "decode_step_cold_ms_p50": float(np.percentile(d["cold_ms"], 50)),
            "decode_step_with_host_ms_p50": float(np.percentile(d["with_host_ms"], 50)),
            "host_prep_ms_p50": float(np.percentile(d["host_ms"], 50)),
            "host_prep_ms_p90": float(np.percentile(d["host_ms"], 90)),
            "stage_wait_ms_p50": float(np.percentile(d["wait_ms"], 50)),
            "kv_tokens_per_s": float(tokens.sum() / (ms.sum() / 1e3)),
            "logical_tb_s": float(tokens.sum() * LAYER_TOKEN_BYTES / (ms.sum() / 1e3) / 1e12),
        }
        out.update(extra)
        return out

    rec = leg(p, {
        "workload": "continuous-batching trace: <=64 rows, one layer 32x128 FP16, 36,864-block pool, "
                    "prompts U{50..8000}, answers U{1..1000}, 2,000-token prefix shared by 125 ref-counted blocks",
        "steps": steps,
        "cold_steps": int(len(p["cold_ms"])),
        "logical_kv_tokens_per_step_mean": float(tokens.mean()),
        "joins": p["joins"],
        "fill_ms_total": float(p["fill_ms"].sum()),
        "pool_drained": True,
        "host_prep_note": "one pkv_grow_rows call, staging into pinned memory and the async uploads; "
                          "the synthetic draws are not counted, and the wait for a free staging buffer of the "
                          "4-deep ring (the host running ahead of the GPU) is stage_wait_ms",
    })
    rec["shared_prefix_decode"] = leg(s, {
        "sharing_rows_per_step_mean": float(sharers.mean()),
        "read_kv_tokens_per_step_mean": float(physical.mean()),
        "read_tb_s": float(physical.sum() * LAYER_TOKEN_BYTES / (s["step_ms"].sum() / 1e3) / 1e12),
        "speedup_vs_plain": float(p["step_ms"].sum() / s["step_ms"].sum()),
    })
    return rec


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-trace", action="store_true", help="skip the continuous-batching trace")
    ap.add_argument("--no-extra", action="store_true", help="skip the long-context step and the block copies")
    ap.add_argument("--trace-steps", type=int, default=300)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (a known-size kernel for "
                         "calibrating HBM byte counters)")
    return ap.parse_args()


def measure_bandwidth(torch, pkv, cache, tables, tlen, stream):
    """Achievable read bandwidth on this machine, from the probes in
    libpkv_probe.so: the (block, layer) slabs one decode step of the average
    mix reads (the same 256 KiB slabs, every layer in turn, one workgroup per
    slab), and a plain 2 GiB stream; each with the streaming (non-temporal)
    cache policy the decode kernels use and with ordinary loads."""
    from paged_kv_cache_pkv_amd import probe

    pool = cache.pool
    dev = pool.device
    NL, H = int(pool.shape[1]), int(pool.shape[3])
    slab_bytes = 2 * H * 16 * 128 * 2
    ids = np.concatenate([tables[r, :tlen[r]] for r in range(tables.shape[0])]).astype(np.int64)
    idx = torch.from_numpy(np.stack([ids * NL + l for l in range(NL)]).astype(np.int32)).to(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        fn(0)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    slab_nt = timed(lambda i: probe.slab_read(pool, idx[i % NL], slab_bytes, sink, True, stream), 2 * NL)
    slab_pl = timed(lambda i: probe.slab_read(pool, idx[i % NL], slab_bytes, sink, False, stream), 2 * NL)
    buf = torch.empty((1 << 31) - 4096, dtype=torch.uint8, device=dev)
    stream_nt = timed(lambda i: probe.stream_read(buf, sink, True, stream), 10)
    stream_pl = timed(lambda i: probe.stream_read(buf, sink, False, stream), 10)
    nslab = float(len(ids) * slab_bytes)
    del buf
    return {
        "probe": "libpkv_probe.so (include/pkv_probe.h)",
        "slab_read_gb_s": nslab / (slab_nt / 1e3) / 1e9,
        "slab_read_plain_gb_s": nslab / (slab_pl / 1e3) / 1e9,
        "slab_read_note": f"{len(ids)} (block, layer) slabs of {slab_bytes} B per launch: the K and V one "
                          "average-mix decode launch reads, non-temporal (plain: ordinary loads)",
        "stream_read_gb_s": ((1 << 31) - 4096) / (stream_nt / 1e3) / 1e9,
        "stream_read_plain_gb_s": ((1 << 31) - 4096) / (stream_pl / 1e3) / 1e9,
    }


def own_slab_ceiling(torch, stream, parts, batch, NL, reps=2):
    """Read rate of the slab probe over the (block, layer) slabs that one decode
    launch of a given cache layout reads, every layer in turn with the
    non-temporal policy: parts = [(tensor, slab_bytes)], each tensor
    [blocks][NL][...] with one contiguous slab of slab_bytes per (block,
    layer) (for example the 8-bit codes and their scales).  GB/s over whole
    slabs."""
    from paged_kv_cache_pkv_amd import probe

    dev = parts[0][0].device
    nblk = [-(-int(L) // 16) for L in batch.context_lens]
    ids = np.concatenate([batch.block_tables[r, :nblk[r]] for r in range(batch.rows)]).astype(np.int64)
    idx = torch.from_numpy(np.stack([ids * NL + l for l in range(NL)]).astype(np.int32)).to(dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def one(layer):
        for t, sb in parts:
            probe.slab_read(t, idx[layer], sb, sink, True, stream)

    one(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps * NL):
        one(i % NL)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * NL)
    return len(ids) * sum(sb for _, sb in parts) / (ms / 1e3) / 1e9


def measure_mfma_ceiling(torch, stream, iters=4000, reps=5):
    """Sustained FP16 matrix-core rate on this machine, from the probe in
    libpkv_probe.so: every SIMD kept busy with independent
    v_mfma_f32_32x32x16_f16 chains for about a millisecond per launch, the
    clock settling where sustained matrix work holds it."""
    from paged_kv_cache_pkv_amd import probe

    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe.mfma_f16(iters, sink, stream)
    torch.cuda.synchronize()
    e0.record(stream)
    flops = sum(probe.mfma_f16(iters, sink, stream) for _ in range(reps))
    e1.record(stream)
    torch.cuda.synchronize()
    return {"probe": "libpkv_probe.so pkv_probe_mfma_f16 (include/pkv_probe.h)",
            "mfma_f16_tflops": flops / (e0.elapsed_time(e1) / 1e3) / 1e12,
            "note": f"{reps} launches of {iters} rounds of 4 independent MFMA chains per wave, 16 waves per CU"}


def measure_block_copies(torch, pkv, cache, free_ids, stream, n=64, reps=10):
    """Copy-on-write and swap of whole 8 MiB blocks (all 32 layers) among free
    blocks of the decode pool: n pairs per copy launch, n blocks per swap."""
    if len(free_ids) < 2 * n:
        return None
    dev = cache.pool.device
    bb = pkv.block_bytes(cache)
    src = torch.from_numpy(np.ascontiguousarray(free_ids[:n], dtype=np.int32)).to(dev)
    dst = torch.from_numpy(np.ascontiguousarray(free_ids[n:2 * n], dtype=np.int32)).to(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    pkv.copy_blocks(cache, src, dst, stream=stream)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        pkv.copy_blocks(cache, src, dst, stream=stream)
    ev[1].record(stream)
    host = torch.empty(n * bb, dtype=torch.uint8, pin_memory=True)
    out_ids, in_ids = free_ids[:n], free_ids[n:2 * n]
    pkv.swap_out(cache, out_ids, host, stream=stream)
    pkv.swap_in(cache, host, in_ids, stream=stream)
    torch.cuda.synchronize()
    ev[2].record(stream)
    for _ in range(reps):
        pkv.swap_out(cache, out_ids, host, stream=stream)
    ev[3].record(stream)
    for _ in range(reps):
        pkv.swap_in(cache, host, in_ids, stream=stream)
    ev[4].record(stream)
    torch.cuda.synchronize()
    copy_ms = ev[0].elapsed_time(ev[1]) / reps
    out_ms = ev[2].elapsed_time(ev[3]) / reps
    in_ms = ev[3].elapsed_time(ev[4]) / reps
    moved = n * bb
    copy_gbs = 2 * moved / (copy_ms / 1e3) / 1e9  # each byte read once and written once
    return {
        "workload": f"{n} whole blocks of {bb >> 20} MiB (32 layers x 32 heads) among free blocks of the decode pool",
        "copy_on_write_us": copy_ms * 1e3,
        "copy_roofline": {"bound": "hbm", "achieved": copy_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": copy_gbs / HBM_PEAK_GBS, "traffic": None,
                          "kernel": "copy_blocks_kernel (read + write bytes)"},
        "swap_out_gb_s": moved / (out_ms / 1e3) / 1e9,
        "swap_in_gb_s": moved / (in_ms / 1e3) / 1e9,
        "swap_note": "device <-> pinned host over the host link, one DMA copy per run of consecutive ids",
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_tiny(torch, pkv, dev, stream, reps=50, cold_reps=10):
    """The tiny decode configuration (4 rows with contexts 17/40/100/256, one
    layer, 64-block pool): append + decode per step, also as the one fused
    call.  Its 6.8 MB stay in the caches, so this is the path's launch
    latency, not a bandwidth figure; the cold-cache figure scrubs the 256 MB
    last-level cache (a 512 MB streaming write) before each timed step."""
    from workloads import SCALE, c1_tiny

    b = c1_tiny(seed=0)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    pool = d(b.pool)
    cache = pkv.PagedCache(pool)
    tables, lens, pos, rot = d(b.block_tables), d(b.context_lens), d(b.positions), d(b.request_of_token)
    q, k, v = d(b.q[0]), d(b.k_new[0]), d(b.v_new[0])
    maxL = int(b.context_lens.max())
    ws = torch.empty(pkv.decode_workspace_size(cache, b.rows, maxL), dtype=torch.uint8, device=dev)
    out = torch.empty((b.rows, 32, 128), dtype=torch.float16, device=dev)

    def step():
        pkv.append(cache, 0, k, v, pos, rot, tables, stream=stream)
        pkv.decode_attention(cache, 0, out, q, tables, lens, maxL, SCALE, ws, stream=stream)

    def fused():
        pkv.decode_attention_append(cache, 0, out, q, k, v, tables, lens, maxL, SCALE, ws, stream=stream)

    def warm(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    def cold(fn):
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        us = []
        for _ in range(cold_reps):
            scrub.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        del scrub
        return float(np.median(us))

    return {"workload": "4 rows, contexts 17/40/100/256, one layer, 64-block pool: append + decode",
            "us_per_step": warm(step), "us_per_step_fused": warm(fused),
            "cold_cache_us_per_step": cold(step), "cold_cache_us_per_step_fused": cold(fused),
            "kv_tokens": int(b.context_lens.sum())}


def measure_long_context(torch, pkv, cache, stream, steps=5, warm=2):
    """The 13 x 8,192-token long-context step (seed 2) on the 32-layer pool:
    per layer, append the 13 new tokens and run decode attention."""
    from workloads import SCALE, c3_long_context

    b = c3_long_context(seed=2, with_pool=False)
    dev = cache.pool.device
    NL = int(cache.desc.num_layers)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    tables, lens, pos, rot = d(b.block_tables), d(b.context_lens), d(b.positions), d(b.request_of_token)
    q, k, v = d(b.q[0]), d(b.k_new[0]), d(b.v_new[0])
    maxL = int(b.context_lens.max())
    ws = torch.empty(pkv.decode_workspace_size(cache, b.rows, maxL), dtype=torch.uint8, device=dev)
    out = torch.empty((b.rows, int(cache.desc.num_heads), 128), dtype=torch.float16, device=dev)

    def step():
        for l in range(NL):
            pkv.append(cache, l, k, v, pos, rot, tables, stream=stream)
            pkv.decode_attention(cache, l, out, q, tables, lens, maxL, SCALE, ws, stream=stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tokens = float(b.context_lens.sum())
    return {
        "workload": "13 rows x 8,192 tokens, 32 layers (append + decode per layer), 60 GB pool",
        "ms_per_step": ms,
        "kv_tokens_per_s": tokens / (ms / 1e3),
        "hbm_tb_s": tokens * STEP_TOKEN_BYTES / (ms / 1e3) / 1e12,
        "hbm_frac_of_peak": tokens * STEP_TOKEN_BYTES / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
    }


def measure_gqa(torch, pkv, batch, stream, kv_heads=8, q_heads=32, steps=10, warm=3, payload=None, counted="gqa"):
    """Grouped-query decode: the average mix's tables and lengths over a
    32-layer pool of kv_heads KV heads, q_heads query heads (8 and 32: groups
    of 4; 4 and 32: groups of 8); per layer one decode launch.  Bytes = K and
    V of the KV heads per token.  With `payload` (a list), layer 0's first
    output and the blocks it read are kept for the oracle leg.  `counted`:
    this shape's key in the committed counter summary ("gqa" for groups of 4,
    "gqa8" for groups of 8), or None."""
    from workloads import SCALE, fill_normal_fp16_device

    NB, NL = 7152, 32
    dev = torch.device("cuda", 0)
    pool = torch.empty((NB, NL, 2, kv_heads, 16, 128), dtype=torch.int16, device=dev)
    fill_normal_fp16_device(pool, seed=3003)
    cache = pkv.PagedCache(pool)
    tables = torch.from_numpy(batch.block_tables).to(dev)
    lens = torch.from_numpy(batch.context_lens.astype(np.int32)).to(dev)
    R = batch.rows
    maxL = int(batch.context_lens.max())
    rng = np.random.default_rng(3004)
    q = torch.from_numpy(rng.standard_normal((NL, R, q_heads, 128), dtype=np.float32).astype(np.float16)).to(dev)
    out = torch.empty((R, q_heads, 128), dtype=torch.float16, device=dev)
    ws = torch.empty(pkv.decode_workspace_size_gqa(cache, q_heads, R, maxL), dtype=torch.uint8, device=dev)
    if payload is not None:
        nblk = [-(-int(L) // 16) for L in batch.context_lens]
        ids = np.unique(np.concatenate([batch.block_tables[r, :nblk[r]] for r in range(R)]))
        slab = pool[torch.from_numpy(ids.astype(np.int64)).to(dev), 0].cpu().numpy().view(np.uint16)
        pkv.decode_attention_gqa(cache, q_heads, 0, out, q[0], tables, lens, maxL, SCALE, ws, stream=stream)
        torch.cuda.synchronize()
        payload.append((ids, slab, q[0].cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16),
                        batch.block_tables, batch.context_lens, q_heads // kv_heads))

    def step():
        for l in range(NL):
            pkv.decode_attention_gqa(cache, q_heads, l, out, q[l], tables, lens, maxL, SCALE, ws, stream=stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the same step with each row's new token appended in the decode launch
    kn = torch.from_numpy(rng.standard_normal((R, kv_heads, 128), dtype=np.float32).astype(np.float16)).to(dev)
    vn = torch.from_numpy(rng.standard_normal((R, kv_heads, 128), dtype=np.float32).astype(np.float16)).to(dev)

    def step_append():
        for l in range(NL):
            pkv.decode_attention_append_gqa(cache, q_heads, l, out, q[l], kn, vn, tables, lens, maxL, SCALE, ws,
                                            stream=stream)

    step_append()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        step_append()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_append = e0.elapsed_time(e1) / steps
    tokens = float(batch.context_lens.sum())
    kv_bytes = tokens * NL * 2 * kv_heads * 128 * 2
    own = own_slab_ceiling(torch, stream, [(pool, 2 * kv_heads * 16 * 128 * 2)], batch, NL)
    del pool
    return {
        "ms_per_step_with_fused_append": ms_append,
        "workload": f"average-mix decode with grouped-query attention: {R} rows x {NL} layers, {kv_heads} KV heads, "
                    f"{q_heads} query heads, FP16, {NB} blocks of 16",
        "ms_per_step": ms,
        "kv_tokens_per_s": tokens / (ms / 1e3),
        "hbm_tb_s": kv_bytes / (ms / 1e3) / 1e12,
        "hbm_frac_of_peak": kv_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "traffic_bytes_per_launch": fp8_gqa_traffic(counted) if counted else None,
        "own_layout_slab_read_gb_s": own,
        "frac_of_own_layout_read": kv_bytes / (ms / 1e3) / 1e9 / own,
        "own_layout_note": f"the slab probe over this pool's (block, layer) slabs of {2 * kv_heads * 4} KiB",
    }


def measure_fp8(torch, pkv, batch, stream, steps=10, warm=3):
    """Decode step over an 8-bit cache: the average mix's 32 rows over a
    32-layer, 7,152-block pool of FP8 E4M3 codes with one fp32 scale per
    (token, head); per layer the 8-bit append of the 32 new tokens fused into
    decode (and, for comparison, the append as a launch of its own).  Bytes = codes + scales of every cached token (8,448 B per token
    and layer).  Codes are seeded random finite values: this leg times the
    kernels; parity and the quality cost are checked by the tests."""
    from workloads import SCALE

    NB, NL, H = 7152, 32, 32
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4004)
    codes = torch.empty((NB, NL, 2, H, 16, 128), dtype=torch.uint8, device=dev)
    flat = codes.view(-1)
    chunk = 1 << 30
    for st in range(0, flat.numel(), chunk):
        seg = flat[st:st + chunk]
        seg.random_(0, 126, generator=gen)  # finite magnitudes; 0x7E = 448 is the largest
        seg.bitwise_or_(torch.randint(0, 2, seg.shape, dtype=torch.uint8, device=dev, generator=gen) << 7)
    scales = torch.empty((NB, NL, 2, H, 16), dtype=torch.float32, device=dev).uniform_(0.002, 0.006, generator=gen)
    cache = pkv.PagedCache8(codes, scales)
    R = batch.rows
    tables = torch.from_numpy(batch.block_tables).to(dev)
    lens = torch.from_numpy(batch.context_lens.astype(np.int32)).to(dev)
    pos = torch.from_numpy((batch.context_lens - 1).astype(np.int32)).to(dev)
    rot = torch.arange(R, dtype=torch.int32, device=dev)
    maxL = int(batch.context_lens.max())
    q = torch.from_numpy(batch.q.view(np.int16)).to(dev)
    k = torch.from_numpy(batch.k_new.view(np.int16)).to(dev)
    v = torch.from_numpy(batch.v_new.view(np.int16)).to(dev)
    out = torch.empty((R, H, 128), dtype=torch.float16, device=dev)
    ws = torch.empty(pkv.decode_workspace_size_fp8(cache, R, maxL), dtype=torch.uint8, device=dev)

    def step(fused=True):
        for l in range(NL):
            if fused:
                pkv.decode_attention_append_fp8(cache, l, out, q[l], k[l], v[l], tables, lens, maxL, SCALE, ws,
                                                stream=stream)
            else:
                pkv.append_fp8(cache, l, k[l], v[l], pos, rot, tables, stream=stream)
                pkv.decode_attention_fp8(cache, l, out, q[l], tables, lens, maxL, SCALE, ws, stream=stream)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    e0.record(stream)
    for _ in range(steps):
        step(fused=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = e0.elapsed_time(e1) / steps
    # the decode launch alone (decode + merge kernels), layers in turn
    launches = 4 * NL
    e0.record(stream)
    for i in range(launches):
        pkv.decode_attention_fp8(cache, i % NL, out, q[i % NL], tables, lens, maxL, SCALE, ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / launches
    tokens = float(batch.context_lens.sum())
    nbytes = tokens * NL * 2 * H * (128 + 4)
    layer_bytes = nbytes / NL
    own = own_slab_ceiling(torch, stream, [(codes, 2 * H * 16 * 128), (scales, 2 * H * 16 * 4)], batch, NL)
    del codes, scales, cache
    return {
        "workload": f"average-mix decode step over an 8-bit cache: {R} rows x {NL} layers, {H} heads x 128, FP8 E4M3 "
                    f"codes + one fp32 scale per (token, head), {NB} blocks of 16 (append + decode per layer)",
        "ms_per_step": ms,
        "step_path": "per layer one pkv_decode_attention_append_fp8 call",
        "unfused_ms_per_step": ms_unfused,
        "kv_tokens_per_s": tokens / (ms / 1e3),
        "hbm_tb_s": nbytes / (ms / 1e3) / 1e12,
        "hbm_frac_of_peak": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "vs_fp16_bytes": (128 + 4) / 256,
        "decode_avg_launch_us": launch_ms * 1e3,
        "decode_hbm_tb_s": layer_bytes / (launch_ms / 1e3) / 1e12,
        "decode_frac_of_peak": layer_bytes / (launch_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "decode_traffic_bytes_per_launch": fp8_gqa_traffic("fp8"),
        "own_layout_slab_read_gb_s": own,
        "decode_frac_of_own_layout_read": layer_bytes / (launch_ms / 1e3) / 1e9 / own,
        "own_layout_note": "the slab probe over the codes' 128 KiB and the scales' 4 KiB (block, layer) slabs",
    }


# ---------------- oracle leg (CPU baseline and parity), run in spawned worker processes
# Each worker is a fresh interpreter (spawn: the GPU process is never forked
# into a worker) with BLAS limited to one thread; the read-back blocks sit in
# one shared-memory segment that every worker maps.
_W = {}


def _oracle_worker_init(shm_name, shape, ids, tables, lens, q_bits):
    from multiprocessing import shared_memory

    import threadpoolctl

    threadpoolctl.threadpool_limits(1)
    shm = shared_memory.SharedMemory(name=shm_name)
    _W["shm"] = shm
    _W["slab"] = np.ndarray(shape, dtype=np.uint16, buffer=shm.buf)  # [layers, blocks, 2, H, 16, D]
    _W["index"] = {int(b): i for i, b in enumerate(ids)}
    _W["tables"], _W["lens"], _W["q"] = tables, lens, q_bits       # q: [layers, R, H, D]


def _oracle_task(li, r):
    """fp64 oracle decode of row r on sampled layer li: the gather through the
    block table, then softmax(q K^T / sqrt(128)) V."""
    import oracle.paged as opaged
    from workloads import SCALE

    slab, index = _W["slab"][li], _W["index"]

    class Blocks:
        def __getitem__(self, b):
            return slab[index[int(b)]]

    out = opaged.decode(Blocks(), _W["q"][li], _W["tables"], _W["lens"], SCALE, rows=[r])[0]
    return li, r, out


def _noop(x):
    return x


def oracle_cpu_baseline(args, sample, tables, lens, q_bits, gpu_outs, layer_names):
    """Time the fp64 oracle on the machine's host cores over (row, layer) tasks of
    the benchmark's first step (the sampled layers' blocks were read back
    before any kernel ran and the oracle appended the step's tokens itself),
    for about args.cpu_seconds of wall time.  The first pass over every task
    is also compared with the GPU's outputs of that step."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import resource
    from multiprocessing import shared_memory

    from tests.tolerance import compare

    ids, slab, t_d2h = sample
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    shm = shared_memory.SharedMemory(create=True, size=slab.nbytes)
    try:
        np.ndarray(slab.shape, dtype=np.uint16, buffer=shm.buf)[...] = slab
        ctx = mp.get_context("spawn")
        R = len(lens)
        tasks = [(li, r) for li in range(slab.shape[0]) for r in range(R)]
        tok = {(li, r): int(lens[r]) for li, r in tasks}
        cpu0 = resource.getrusage(resource.RUSAGE_CHILDREN)
        with cf.ProcessPoolExecutor(workers, mp_context=ctx, initializer=_oracle_worker_init,
                                    initargs=(shm.name, slab.shape, ids, tables, lens, q_bits)) as ex:
            list(ex.map(_noop, range(4 * workers)))  # every worker started and initialised
            t0 = time.perf_counter()
            pending, done, n_sub, first = set(), 0, 0, {}
            tokens = 0
            while True:
                while len(pending) < 2 * workers and (time.perf_counter() - t0 < args.cpu_seconds
                                                      or n_sub < len(tasks)):
                    pending.add(ex.submit(_oracle_task, *tasks[n_sub % len(tasks)]))
                    n_sub += 1
                if not pending:
                    break
                fin, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
                for f in fin:
                    li, r, out = f.result()
                    tokens += tok[(li, r)]
                    done += 1
                    first.setdefault((li, r), out)
            wall = time.perf_counter() - t0
        cpu1 = resource.getrusage(resource.RUSAGE_CHILDREN)
    finally:
        shm.close()
        shm.unlink()
    busy = (cpu1.ru_utime + cpu1.ru_stime) - (cpu0.ru_utime + cpu0.ru_stime)
    parity = {"layers": layer_names, "rows": R, "max_abs": 0.0, "max_rel": 0.0, "bad": 0}
    for (li, r), ref in first.items():
        c = compare(gpu_outs[li][r], ref)
        parity["max_abs"] = max(parity["max_abs"], c["max_abs"])
        parity["max_rel"] = max(parity["max_rel"], c["max_rel"])
        parity["bad"] += c["bad"] + c["nan"]
    parity["pass"] = parity["bad"] == 0
    nl = 32
    baseline = {
        "value": (tokens / nl) / wall, "unit": "KV-tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"fp64 NumPy oracle decode of (row, layer) tasks of the average-mix step (rows 0..{R - 1}, "
                  f"layers {layer_names}), {done} tasks = {tokens} one-layer KV-tokens in {wall:.1f} s on "
                  f"{workers} worker processes, BLAS at 1 thread each; value = one-layer tokens / 32 / s",
        "cpu_seconds": busy, "wall_seconds": wall, "cpu_time_over_wall": busy / wall,
        "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
        "d2h_readback_s": t_d2h,
        "d2h_note": "the sampled layers' blocks copied to host memory before any kernel ran; not in the timed run",
    }
    return baseline, parity


def gqa_parity(payload):
    """A grouped-query leg's first decode (layer 0, G = 4 or 8, weights
    rounded to FP16 before P.V) against the fp64 oracle."""
    import oracle.paged as opaged
    from tests.tolerance import compare
    from workloads import SCALE

    ids, slab, q0, out0, tables, lens, group = payload
    index = {int(b): i for i, b in enumerate(ids)}

    class Blocks:
        def __getitem__(self, b):
            return slab[index[int(b)]]

    ref = opaged.decode(Blocks(), q0, tables, lens, SCALE, group=group)
    c = compare(out0.view(np.float16).astype(np.float64), ref)
    return {"layer": 0, "rows": int(len(lens)), "group": group, "max_abs": c["max_abs"], "max_rel": c["max_rel"],
            "bad": c["bad"] + c["nan"], "pass": c["bad"] + c["nan"] == 0}


def log(args, msg):
    if not args.quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would serve its own requests or its own heads with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_pkv_amd as pkv
    from workloads import SCALE, c2_average_mix, fill_normal_fp16_device

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    NB, NL, H, D = 7152, 32, 32, 128
    batch = c2_average_mix(seed=args.seed, with_pool=False)
    R = batch.rows
    stride = batch.bt_stride
    UNFUSED_STEPS = 5  # after the timed steps: the same step with the append as its own launch
    total_steps = args.warmup + args.steps + UNFUSED_STEPS
    lens0 = batch.context_lens.astype(np.int64)
    max_ctx = int(lens0.max()) + total_steps
    if -(-max_ctx // 16) > stride:
        raise SystemExit("table stride too small for the run length")

    log(args, f"allocating pool {NB}x{NL}x2x{H}x16x{D} FP16 ({NB * NL * 2 * H * 16 * D * 2 / 1e9:.1f} GB)")
    pool_d = torch.empty((NB, NL, 2, H, 16, D), dtype=torch.int16, device=dev)
    fill_normal_fp16_device(pool_d, seed=1000 + args.seed)
    cache = pkv.PagedCache(pool_d)

    # host block pool: shuffled free list, rows allocated in order
    bp = pkv.BlockPool(NB, batch.free_list)
    tables = np.zeros((R, stride), dtype=np.int32)
    tlen = np.zeros(R, dtype=np.int32)
    tlen[:] = [bp.grow(tables[r], 0, int(lens0[r])) for r in range(R)]
    for r in range(R):  # the C++ pool hands out the ids the generator's LIFO reading predicts
        assert np.array_equal(tables[r, :tlen[r]], batch.block_tables[r, :tlen[r]])

    q_d = torch.from_numpy(batch.q.view(np.int16)).to(dev)         # [NL, R, H, D]
    k_d = torch.from_numpy(batch.k_new.view(np.int16)).to(dev)
    v_d = torch.from_numpy(batch.v_new.view(np.int16)).to(dev)
    out_d = torch.empty((NL, R, H, D), dtype=torch.float16, device=dev)
    rot_d = torch.arange(R, dtype=torch.int32, device=dev)
    tables_d = torch.empty((R, stride), dtype=torch.int32, device=dev)
    lens_d = torch.empty(R, dtype=torch.int32, device=dev)
    pos_d = torch.empty(R, dtype=torch.int32, device=dev)
    ws_bytes = pkv.decode_workspace_size(cache, R, max_ctx)
    ws_d = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # pinned staging, one set per step so the host never overwrites a buffer in flight
    stage = [torch.empty(R * stride + 2 * R, dtype=torch.int32, pin_memory=True) for _ in range(total_steps)]

    # ---------------- oracle-leg input: two layers' blocks read back before any kernel touches the pool
    ORACLE_LAYERS = (0, NL - 1)
    cpu_sample = None
    if not args.no_cpu_baseline:
        ids = np.unique(np.concatenate([tables[r, :tlen[r]] for r in range(R)]))
        torch.cuda.synchronize()
        t_d2h = time.perf_counter()
        ids_d = torch.from_numpy(ids.astype(np.int64)).to(dev)
        slab = np.stack([pool_d[ids_d, l].cpu().numpy().view(np.uint16) for l in ORACLE_LAYERS])
        t_d2h = time.perf_counter() - t_d2h
        cpu_sample = (ids, slab, t_d2h)

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def host_step(k):
        """Grow tables for this step's new token (one pkv_grow_rows call), stage the upload."""
        lens = lens0 + k
        if bp.grow_rows(tables, tlen, lens) != R:
            raise SystemExit("block pool exhausted")
        buf = stage[k]
        a = buf.numpy()
        a[: R * stride] = tables.reshape(-1)
        a[R * stride: R * stride + R] = lens
        a[R * stride + R:] = lens - 1
        tables_d.copy_(buf[: R * stride].view(R, stride), non_blocking=True)
        lens_d.copy_(buf[R * stride: R * stride + R], non_blocking=True)
        pos_d.copy_(buf[R * stride + R:], non_blocking=True)
        return int(lens.sum())

    def gpu_step(fused=True):
        """Per layer: the step's append and decode attention.  By default one
        fused call (the range holding each row's new token appends it);
        fused=False runs pkv_append then pkv_decode_attention."""
        for l in range(NL):
            if fused:
                pkv.decode_attention_append(cache, l, out_d[l], q_d[l], k_d[l], v_d[l], tables_d, lens_d, max_ctx,
                                            SCALE, ws_d, stream=stream)
            else:
                pkv.append(cache, l, k_d[l], v_d[l], pos_d, rot_d, tables_d, stream=stream)
                pkv.decode_attention(cache, l, out_d[l], q_d[l], tables_d, lens_d, max_ctx, SCALE, ws_d,
                                     stream=stream)

    log(args, f"rows={R} sum_context={int(lens0.sum())} max_context={int(lens0.max())} ws={ws_bytes}")
    step0_outs = None
    for k in range(args.warmup):
        host_step(k)
        gpu_step()
        if k == 0:
            torch.cuda.synchronize()
            step0_outs = [out_d[l].cpu().numpy().view(np.uint16).view(np.float16).astype(np.float64)
                          for l in ORACLE_LAYERS]
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    tokens = 0
    step_tokens = []
    t_start.record(stream)
    wall0 = time.perf_counter()
    step_ev = events(args.steps + 1)
    for i, k in enumerate(range(args.warmup, args.warmup + args.steps)):
        st = host_step(k)
        tokens += st
        step_tokens.append(st)
        step_ev[i].record(stream)  # after the step's uploads are queued: brackets the 32 layer calls
        gpu_step()
    step_ev[args.steps].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = t_start.elapsed_time(t_end)
    log(args, f"timed {args.steps} steps: {elapsed_ms:.2f} ms (wall {wall * 1e3:.1f} ms)")

    # the same step with pkv_append as a launch of its own, for comparison (not the headline)
    u0, u1 = events(2)
    unfused_tokens = 0
    u0.record(stream)
    for k in range(args.warmup + args.steps, total_steps):
        unfused_tokens += host_step(k)
        gpu_step(fused=False)
    u1.record(stream)
    torch.cuda.synchronize()
    unfused_ms = u0.elapsed_time(u1) / UNFUSED_STEPS

    ms_per_step = elapsed_ms / args.steps
    step_ms = [step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)]
    value = tokens / (elapsed_ms / 1e3)
    # The dominant kernel is the decode call (split + merge launches, the
    # append fused).  Its average duration: the events bracketing each step's
    # 32 back-to-back calls (and nothing else) over the timed steps, / 32.
    launches = NL * args.steps
    dec_avg_ms = float(np.sum(step_ms)) / launches
    bytes_per_decode = float(np.mean(step_tokens)) * LAYER_TOKEN_BYTES
    achieved = bytes_per_decode / (dec_avg_ms / 1e3) / 1e9
    traffic = counted_traffic()

    blocks = long_ctx = gqa = gqa8 = fp8 = tiny = probe = None
    gqa_payload = [] if cpu_sample is not None else None
    gqa8_payload = [] if cpu_sample is not None else None
    if not args.no_extra:
        probe = measure_bandwidth(torch, pkv, cache, tables, tlen, stream)
        blocks = measure_block_copies(torch, pkv, cache, bp.free_list(), stream)
        long_ctx = measure_long_context(torch, pkv, cache, stream)
        # The 60 GB pool goes back to torch's cache, not to the driver: the
        # later legs' pools are carved from it.  A 60 GB free to the driver
        # slowed every read on the device by about 8% for tens of seconds
        # afterwards (most plausibly the driver clearing the freed memory).
        del pool_d, cache
        gqa = measure_gqa(torch, pkv, batch, stream, payload=gqa_payload)
        gqa8 = measure_gqa(torch, pkv, batch, stream, kv_heads=4, q_heads=32, payload=gqa8_payload, counted="gqa8")
        fp8 = measure_fp8(torch, pkv, batch, stream)
        tiny = measure_tiny(torch, pkv, dev, stream)
    else:
        del pool_d, cache

    prefill = None
    if not args.no_prefill:
        prefill = measure_prefill(torch, pkv, dev, stream)

    trace = None
    checkers = [] if cpu_sample is not None else None
    if not args.no_trace:
        trace = measure_trace(torch, steps=args.trace_steps, checkers=checkers)

    # ---------------- oracle leg: CPU baseline and parity against the fp64 oracle
    cpu_baseline = parity = None
    if cpu_sample is not None:
        log(args, "oracle leg: CPU baseline and parity")
        pos0 = (lens0 - 1).astype(np.int64)
        ids, slab, _ = cpu_sample
        index = {int(bk): i for i, bk in enumerate(ids)}
        for li, l in enumerate(ORACLE_LAYERS):  # the oracle's own append of step 0's tokens
            for r in range(R):
                bk = int(batch.block_tables[r, pos0[r] // 16])
                slab[li, index[bk], 0, :, pos0[r] % 16, :] = batch.k_new[l, r]
                slab[li, index[bk], 1, :, pos0[r] % 16, :] = batch.v_new[l, r]
        q_bits = np.stack([batch.q[l] for l in ORACLE_LAYERS])
        cpu_baseline, parity = oracle_cpu_baseline(args, cpu_sample, batch.block_tables, lens0.astype(np.int32),
                                                   q_bits, step0_outs, list(ORACLE_LAYERS))
        if gqa is not None and gqa_payload:
            gqa["parity"] = gqa_parity(gqa_payload[0])
        if gqa8 is not None and gqa8_payload:
            gqa8["parity"] = gqa_parity(gqa8_payload[0])
        if trace is not None and checkers:
            for name, chk in checkers:
                tot = chk.check(rows=TRACE_CHECK_ROWS)
                tot["rows_per_step"] = len(TRACE_CHECK_ROWS)
                tot["timed_steps_sampled"] = list(TRACE_SAMPLED)
                tot["pass"] = tot["bad"] == 0 and tot["nan"] == 0
                (trace if name == "appending" else trace["shared_prefix_decode"])["parity"] = tot

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "KV-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "step_path": "per layer one pkv_decode_attention_append call (append fused into decode)",
        "unfused_step": {"ms_per_step": unfused_ms,
                         "kv_tokens_per_s": unfused_tokens / (unfused_ms * UNFUSED_STEPS / 1e3),
                         "path": "per layer pkv_append then pkv_decode_attention", "steps": UNFUSED_STEPS},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 storage, f32 accumulation",
        "data": "synthetic",
        "config": {
            "workload": "average-mix decode step: 32 rows x 32 layers, 32 heads x 128, FP16 KV in 7152 blocks of 16",
            "rows": R, "layers": NL, "heads": H, "head_dim": D, "num_blocks": NB,
            "sum_context_tokens_first_step": int((lens0 + args.warmup).sum()), "seed": args.seed,
        },
        "hbm_tb_s": value * STEP_TOKEN_BYTES / 1e12,
        "hbm_frac_of_peak": value * STEP_TOKEN_BYTES / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "pkv_decode_attention_append (split + merge launches, the append fused), one layer",
                     "avg_launch_ms": dec_avg_ms, "bytes_per_launch": bytes_per_decode,
                     "launches_timed": launches,
                     "timing": "events around each timed step's 32 back-to-back layer calls, / 32 (gaps included)",
                     "achievable": probe},
        "wall_s_timed": wall,
        "parity_step0": parity,
        "prefill": prefill,
        "trace": trace,
        "long_context": long_ctx,
        "gqa_decode": gqa,
        "gqa8_decode": gqa8,
        "fp8_decode": fp8,
        "block_copy": blocks,
        "tiny_decode": tiny,
        "cpu_baseline": cpu_baseline,
    }
    if probe and probe.get("slab_read_gb_s"):
        ceiling = probe["slab_read_gb_s"] / 1e3  # TB/s
        rec["roofline"]["frac_of_achievable"] = achieved / probe["slab_read_gb_s"]
        # the grouped-query, 8-bit and long-context decodes against the same measured read ceiling
        for leg, key in (("gqa_decode", "hbm_tb_s"), ("gqa8_decode", "hbm_tb_s"), ("fp8_decode", "hbm_tb_s"),
                         ("long_context", "hbm_tb_s")):
            if rec.get(leg) and rec[leg].get(key):
                rec[leg]["frac_of_achievable"] = rec[leg][key] / ceiling
                rec[leg]["achievable_note"] = "the FP16 average-mix slab probe (256 KiB slabs) as the read ceiling"
    print(json.dumps(rec), flush=True)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(args, f"copy probe: 3 x {args.copy_probe_mib} MiB device-to-device copies done")


if __name__ == "__main__":
    main()
