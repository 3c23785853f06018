"""A decode step and a mixed prefill launch captured in a HIP graph and
replayed: every replay gives the eager calls' bits.

The calls record kernel launches only (no memset or copy nodes), so a
captured step can be replayed by a serving loop; the graph here holds four
layers of decode with the append fused (through the workspace call and the
no-alloc call) and one chunked-prefill launch, replayed three times with
eager work and synchronisations between the replays."""
import numpy as np
import pytest

import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, say, torch_cuda
from workloads import SCALE, build_batch, c5_mixed, fill_normal_fp16_device

pytestmark = pytest.mark.gpu

NL = 4


def test_graph_replays_give_eager_bits():
    torch = torch_cuda()
    lens = np.clip(np.random.default_rng(41).lognormal(6.5, 1.0, 20).astype(np.int64), 1, 5000).tolist()
    R = len(lens)
    b = build_batch("graph", 41, lens, [1] * R, num_blocks=sum(-(-L // 16) for L in lens) + 8, num_layers=NL)
    say(f"graph: {R} rows, {NL} layers, contexts {min(lens)}..{max(lens)}")
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    tables, lens_d = dev(b.block_tables, torch), dev(b.context_lens, torch)
    q, k, v = dev(b.q, torch), dev(b.k_new, torch), dev(b.v_new, torch)
    maxL = max(lens)
    ws = torch.empty(pkv.decode_workspace_size(cache, R, maxL), dtype=torch.uint8, device="cuda")
    out = torch.empty((NL, R, 32, 128), dtype=torch.float16, device="cuda")
    out_na = torch.empty_like(out)
    m = c5_mixed(with_pool=False)
    pool_m = torch.empty((7152, 1, 2, 32, 16, 128), dtype=torch.int16, device="cuda")
    fill_normal_fp16_device(pool_m, seed=42)
    cache_m = pkv.PagedCache(pool_m)
    mt = [dev(x, torch) for x in (m.block_tables, m.query_start, m.context_lens, m.q[0])]
    T, maxq, maxLm = m.total_q, int(m.q_counts.max()), int(m.context_lens.max())
    ws_m = torch.empty(pkv.prefill_workspace_size(cache_m, m.rows, T, maxq, maxLm), dtype=torch.uint8, device="cuda")
    out_m = torch.empty((T, 32, 128), dtype=torch.float16, device="cuda")

    def step():
        for layer in range(NL):
            pkv.decode_attention_append(cache, layer, out[layer], q[layer], k[layer], v[layer], tables, lens_d, maxL,
                                        SCALE, ws)
            pkv.decode_attention_append_noalloc(cache, layer, out_na[layer], q[layer], k[layer], v[layer], tables,
                                                lens_d, maxL, SCALE)
        pkv.chunked_prefill_attention(cache_m, 0, out_m, mt[3], mt[1], mt[0], mt[2], maxq, maxLm, SCALE, ws_m)

    # eager (the fused appends rewrite the same slots with the same bits on every call)
    step()
    torch.cuda.synchronize()
    want, want_m, want_pool = out.clone(), out_m.clone(), pool_d.clone()
    assert torch.equal(out_na.view(torch.int16), want.view(torch.int16))
    # capture, after a warm-up on the capture stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, out_na, out_m):
            t.fill_(0)
        # eager work between replays: the same layers' calls into other outputs
        scratch = torch.empty_like(out[0])
        pkv.decode_attention_append(cache, rep % NL, scratch, q[rep % NL], k[rep % NL], v[rep % NL], tables, lens_d,
                                    maxL, SCALE, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), rep
        assert torch.equal(out_na.view(torch.int16), want.view(torch.int16)), rep
        assert torch.equal(out_m.view(torch.int16), want_m.view(torch.int16)), rep
        assert torch.equal(pool_d, want_pool), rep
