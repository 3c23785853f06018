"""Independent calls on two streams at once give the bits each gives alone.

The library keeps no device state between calls (workspaces are the
caller's), so decode and chunked prefill on different pools, queued on two
streams and running concurrently, must not disturb one another."""
import numpy as np
import pytest

import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, say, torch_cuda
from workloads import SCALE, build_batch, c5_mixed, fill_normal_fp16_device

pytestmark = pytest.mark.gpu


def _decode_setup(torch, seed, heads):
    lens = np.clip(np.random.default_rng(seed).lognormal(6.5, 1.0, 24).astype(np.int64), 1, 6000).tolist()
    b = build_batch(f"streams-{seed}", seed, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=2, num_heads=heads)
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    maxL = max(lens)
    args = dict(tables=dev(b.block_tables, torch), lens=dev(b.context_lens, torch), q=dev(b.q[1], torch),
                k=dev(b.k_new[1], torch), v=dev(b.v_new[1], torch), maxL=maxL,
                ws=torch.empty(max(pkv.decode_workspace_size(cache, len(lens), maxL), 256), dtype=torch.uint8,
                               device="cuda"),
                out=torch.empty((len(lens), heads, 128), dtype=torch.float16, device="cuda"))
    return b, pool_d, cache, args


def _decode(cache, a, stream):
    pkv.decode_attention_append(cache, 1, a["out"], a["q"], a["k"], a["v"], a["tables"], a["lens"], a["maxL"], SCALE,
                                a["ws"], stream=stream)


def test_two_streams_decode_and_prefill():
    torch = torch_cuda()
    say("two streams: decode on two pools and a mixed prefill launch")
    ra = _decode_setup(torch, 31, 32)
    rb = _decode_setup(torch, 32, 8)
    # a mixed prefill batch on a third pool
    m = c5_mixed(with_pool=False)
    pool_m = torch.empty((7152, 1, 2, 32, 16, 128), dtype=torch.int16, device="cuda")
    fill_normal_fp16_device(pool_m, seed=5)
    cache_m = pkv.PagedCache(pool_m)
    mt = dict(tables=dev(m.block_tables, torch), qs=dev(m.query_start, torch), lens=dev(m.context_lens, torch),
              q=dev(m.q[0], torch))
    T, maxq, maxL = m.total_q, int(m.q_counts.max()), int(m.context_lens.max())
    ws_m = torch.empty(pkv.prefill_workspace_size(cache_m, m.rows, T, maxq, maxL), dtype=torch.uint8, device="cuda")
    out_m = torch.empty((T, 32, 128), dtype=torch.float16, device="cuda")

    def prefill(stream):
        pkv.chunked_prefill_attention(cache_m, 0, out_m, mt["q"], mt["qs"], mt["tables"], mt["lens"], maxq, maxL,
                                      SCALE, ws_m, stream=stream)

    # alone, one after another on the default stream (the fused appends rewrite the same slots with the same bits)
    snap_pools = [ra[1].clone(), rb[1].clone()]
    _decode(ra[2], ra[3], None)
    _decode(rb[2], rb[3], None)
    prefill(None)
    torch.cuda.synchronize()
    want = [ra[3]["out"].clone(), rb[3]["out"].clone(), out_m.clone()]
    want_pools = [ra[1].clone(), rb[1].clone()]
    # concurrently: restore the pools, then interleave the calls over two streams, several times over
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        ra[1].copy_(snap_pools[0])
        rb[1].copy_(snap_pools[1])
        for t in (ra[3]["out"], rb[3]["out"], out_m):
            t.fill_(0)
        torch.cuda.synchronize()
        for _ in range(4):
            _decode(ra[2], ra[3], s1)
            prefill(s2)
            _decode(rb[2], rb[3], s1 if rep == 1 else s2)
        torch.cuda.synchronize()
        for got, w, what in zip((ra[3]["out"], rb[3]["out"], out_m), want, ("decode A", "decode B", "prefill")):
            assert torch.equal(got.view(torch.int16), w.view(torch.int16)), (rep, what)
        assert torch.equal(ra[1], want_pools[0]) and torch.equal(rb[1], want_pools[1]), rep
