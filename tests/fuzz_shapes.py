"""Seeded shape fuzzing on the GPU through the same checks as the parity tests.

Not collected by pytest (a script): it draws shapes beyond the committed
cases (longer contexts, more heads, larger prefixes, other group sizes, many
decode rows) and runs them through tests/test_gpu_random_shapes.py's check
functions, the continuous-batching trace check and the no-alloc comparison,
each against the fp64 oracle or the workspace call, until a time budget ends.
Any mismatch raises with the seed that produced it.

    python -m tests.fuzz_shapes --seconds 300 [--seed 777] [--kinds decode,prefill,...]
"""
from __future__ import annotations

import argparse
import time

import numpy as np

import tests.test_gpu_random_shapes as R

KINDS = ("decode", "fp8", "fp8_fused", "prefill", "prefill_groups", "mixed", "prefix", "append", "copies", "trace",
         "noalloc")


def _lens(r, rows, top, mean):
    return [int(x) for x in np.clip(r.lognormal(np.log(mean), 1.0, rows).astype(np.int64), 1, top)]


def one(kind: str, seed: int) -> str:
    r = np.random.default_rng(seed)
    idx = seed % 100000
    if kind == "decode":
        long = r.random() < 0.5
        lens = _lens(r, int(r.integers(1, 9 if long else 65)), 20000 if long else 3000, 6000 if long else 1000)
        hkv = int(r.choice([1, 2, 4, 8] if long else [4, 8, 16, 32]))
        group, fused = int(r.choice([1, 2, 4, 8])), bool(r.integers(0, 2))
        R.test_decode_random_shape(idx, hkv, group, lens, fused)
        return f"kv {hkv} G {group} rows {len(lens)} longest {max(lens)} fused {fused}"
    if kind in ("fp8", "fp8_fused"):
        long = r.random() < 0.4
        lens = _lens(r, int(r.integers(1, 9 if long else 40)), 16000 if long else 4000, 5000 if long else 1300)
        heads = int(r.choice([1, 8, 32] if long else [8, 32, 64]))
        fn = R.test_fp8_decode_random_shape if kind == "fp8" else R.test_fp8_fused_append_decode_random_shape
        fn(idx, heads, lens)
        return f"heads {heads} rows {len(lens)} longest {max(lens)}"
    if kind in ("prefill", "prefill_groups", "mixed"):
        if kind == "prefill":
            hkv, group, rows, top, chunk, p_dec = int(r.choice([1, 2, 4, 8])), int(r.choice([1, 2, 4])), \
                int(r.integers(1, 7)), 10000, 768, 0.3
        elif kind == "prefill_groups":
            group = int(r.choice([3, 5, 6, 8, 16]))
            hkv, rows, top, chunk, p_dec = int(r.choice([1, 2] if group == 16 else [1, 2, 4])), \
                int(r.integers(1, 8)), 6000, 400, 0.3
        else:
            hkv, group, rows, top, chunk, p_dec = int(r.choice([2, 4, 8])), int(r.choice([1, 2, 4])), \
                int(r.integers(8, 65)), 8000, 512, 0.85
        lens = [max(2, L) for L in _lens(r, rows, top, 1500)]
        qc = [1 if r.random() < p_dec else int(r.integers(2, min(L, chunk) + 1)) for L in lens]
        R.test_prefill_random_shape(idx, hkv, group, lens, qc)
        return f"kv {hkv} G {group} rows {rows} queries {sum(qc)} longest {max(lens)}"
    if kind == "prefix":
        P, heads, rows = int(r.integers(1, 201)), int(r.choice([8, 16, 32])), int(r.integers(2, 110))
        lens, shared, lone = [], [], []
        for i in range(rows):
            k = 0 if i == 0 else int(r.choice(3, p=[0.7, 0.2, 0.1]))
            if k == 0:
                lens.append(16 * P + 1 + int(min(r.lognormal(5.5, 1.2), 4000)))
                if i:
                    shared.append(i)
            elif k == 1:
                lens.append(int(np.clip(r.lognormal(6.5, 1.2), 1, 6000)))
            else:
                lens.append(int(r.integers(1, 16 * P + 1)))
                lone.append(i)
        R.test_prefix_decode_random_shape(idx, P, heads, lens, shared, lone)
        return f"P {P} heads {heads} rows {rows} sharing {len(shared)}"
    if kind == "append":
        c = R._append_shapes(seed, 1)[0]
        R.test_append_random_shape(idx, *c[1:])
        return f"heads {c[1]} layers {c[2]} rows {len(c[4])} tokens {sum(c[5])}"
    if kind == "copies":
        layers, heads = int(r.choice([1, 2, 3, 8])), int(r.choice([1, 5, 8, 32]))
        R.test_block_copies_random_shape(idx, layers, heads)
        return f"layers {layers} heads {heads}"
    if kind == "trace":
        return _trace(r, seed)
    if kind == "noalloc":
        return _noalloc(r, seed)
    raise KeyError(kind)


def _trace(r, seed):
    import torch

    from paged_kv_cache_pkv_amd.trace import ContinuousBatchTrace
    from tests.trace_check import TraceChecker

    rows, pre = int(r.integers(2, 17)), int(r.choice([0, 16, 160, 512, 1000]))
    hi = int(r.integers(200, 2500)) if r.random() < 0.8 else int(r.integers(50, 200))
    ans, steps, heads = int(r.integers(1, 80)), int(r.integers(20, 80)), int(r.choice([8, 32]))
    for shared in (False, True):
        nb = rows * (-(-(hi + ans) // 16) + 2) + pre // 16 + 64
        tr = ContinuousBatchTrace(torch, seed=seed % (1 << 20), num_blocks=nb, max_rows=rows, prefix_tokens=pre,
                                  prompt_range=(50, hi), answer_range=(1, ans), heads=heads, shared_decode=shared)
        chk = TraceChecker(tr)
        npre = len(tr.prefix_ids)
        for s in range(steps):
            snap = tr.step()
            chk.record(snap)
            sharers = sum(1 for x in tr.rows if x.shared)
            assert all(tr.pool.ref_count(int(b)) == 1 + sharers for b in tr.prefix_ids)
            assert tr.pool.num_free + sum(x.nblk - x.shared // 16 for x in tr.rows) + npre == nb
            if s % 9 == 4 or s == steps - 1:
                chk.keep(snap)
        tr.drain()
        assert tr.pool.num_free == nb
        tot = chk.check()
        assert tot["bad"] == 0 and tot["nan"] == 0, tot
    return f"rows {rows} prefix {pre} prompts <= {hi} answers <= {ans} steps {steps} heads {heads}"


def _noalloc(r, seed):
    import torch

    import paged_kv_cache_pkv_amd as pkv
    from tests.gpu_util import dev
    from workloads import SCALE, build_batch

    heads, rows = int(r.choice([1, 8, 32, 64])), int(r.integers(1, 65))
    lens = _lens(r, rows, 12000, 1500)
    maxL = max(lens)
    b = build_batch(f"na-{seed}", seed % 100000, lens, [1] * rows, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_heads=heads, stride=-(-maxL // 16) + 1)
    pa, pb = dev(b.pool, torch), dev(b.pool, torch)
    ca, cb = pkv.PagedCache(pa), pkv.PagedCache(pb)
    need = pkv.decode_workspace_size(ca, rows, maxL)
    if need > (64 << 20):
        return f"rows {rows} heads {heads}: {need} B of partials, beyond the no-alloc scratch; not run"
    t = [dev(x, torch) for x in (b.q[0], b.k_new[0], b.v_new[0], b.block_tables, b.context_lens)]
    oa = torch.empty((rows, heads, 128), dtype=torch.float16, device="cuda")
    ob = torch.empty_like(oa)
    pkv.decode_attention_append(ca, 0, oa, *t, maxL, SCALE, torch.empty(max(need, 256), dtype=torch.uint8,
                                                                           device="cuda"))
    pkv.decode_attention_append_noalloc(cb, 0, ob, *t, maxL, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)) and torch.equal(pa, pb), seed
    return f"rows {rows} heads {heads} longest {maxL}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seconds", type=float, default=300.0)
    ap.add_argument("--seed", type=int, default=777)
    ap.add_argument("--kinds", default=",".join(KINDS))
    args = ap.parse_args()
    kinds = [k for k in args.kinds.split(",") if k]
    rng = np.random.default_rng(args.seed)
    t0, n = time.time(), 0
    while time.time() - t0 < args.seconds:
        kind, seed = kinds[n % len(kinds)], int(rng.integers(1 << 30))
        print(f"{kind} seed {seed}", flush=True)  # names the case before it runs
        print(f"  ok: {one(kind, seed)}", flush=True)
        n += 1
    print(f"fuzz done: {n} cases in {time.time() - t0:.0f} s, no mismatch", flush=True)


if __name__ == "__main__":
    main()
