"""Decode parity at full size, in the launch configuration the benchmark times.

The 7,152-block, 32-layer pool (60 GB) is filled on the device with seeded
N(0,1) values; the blocks the sampled layers use are read back before any
kernel runs.  On every layer the library appends the step's tokens and runs
decode attention (pkv_append, then pkv_decode_attention); then the same step
runs again as the benchmark runs it, one pkv_decode_attention_append call per
layer.  The second pass rewrites the same token bits, so both passes must
give the same output bits; the oracle appends the same tokens itself and
recomputes every row of the sampled layers."""
import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, c2_average_mix, c3_long_context, fill_normal_fp16_device

pytestmark = pytest.mark.gpu

NB, NL, H, D = 7152, 32, 32, 128


class Blocks:
    def __init__(self, ids, slab):
        self.index = {int(b): i for i, b in enumerate(ids)}
        self.slab = slab

    def __getitem__(self, b):
        return self.slab[self.index[int(b)]]


def _run(batch, layers, seed, all_layer_rows=()):
    """Check every row of `layers`, and every layer of the rows in `all_layer_rows`."""
    torch = torch_cuda()
    dev = torch.device("cuda", 0)
    pool = torch.empty((NB, NL, 2, H, 16, D), dtype=torch.int16, device=dev)
    fill_normal_fp16_device(pool, seed=seed)
    R = batch.rows
    nblk = [-(-int(L) // 16) for L in batch.context_lens]
    ids = np.unique(np.concatenate([batch.block_tables[r, :nblk[r]] for r in range(R)]))
    ids_d = torch.from_numpy(ids.astype(np.int64)).to(dev)
    before = {l: pool[ids_d, l].cpu().numpy().view(np.uint16) for l in layers}
    # the few rows checked on every layer: their own blocks, all layers
    row_ids = np.unique(np.concatenate([batch.block_tables[r, :nblk[r]] for r in all_layer_rows])) if all_layer_rows \
        else np.zeros(0, dtype=np.int32)
    row_slab = pool[torch.from_numpy(row_ids.astype(np.int64)).to(dev)].cpu().numpy().view(np.uint16) \
        if all_layer_rows else None
    cache = pkv.PagedCache(pool)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    tables, lens, pos = t(batch.block_tables), t(batch.context_lens), t(batch.positions)
    rot = t(batch.request_of_token)
    maxL = int(batch.context_lens.max())
    ws = torch.empty(pkv.decode_workspace_size(cache, R, maxL), dtype=torch.uint8, device=dev)
    out = torch.empty((NL, R, H, D), dtype=torch.float16, device=dev)
    for l in range(NL):
        pkv.append(cache, l, t(batch.k_new[l]), t(batch.v_new[l]), pos, rot, tables)
        pkv.decode_attention(cache, l, out[l], t(batch.q[l]), tables, lens, maxL, SCALE, ws)
    fused = torch.empty_like(out)
    for l in range(NL):
        pkv.decode_attention_append(cache, l, fused[l], t(batch.q[l]), t(batch.k_new[l]), t(batch.v_new[l]), tables,
                                    lens, maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), out.view(torch.int16)), "appending decode differs from append + decode"
    say(f"  {batch.name}: the appending decode gives the same bits as append + decode on all {NL} layers")
    got = fused.cpu().numpy().astype(np.float64)
    for l in layers:
        slab = before[l].copy()
        index = {int(b): i for i, b in enumerate(ids)}
        for r in range(R):  # the oracle's own append of this layer's new tokens
            b, s = opaged.locate(batch.block_tables[r], int(batch.positions[r]))
            slab[index[b], 0, :, s, :] = batch.k_new[l, r]
            slab[index[b], 1, :, s, :] = batch.v_new[l, r]
        ref = opaged.decode(Blocks(ids, slab), batch.q[l], batch.block_tables, batch.context_lens, SCALE)
        s = assert_close(got[l], ref, f"{batch.name} layer {l}")
        say(f"  {batch.name} layer {l}: {s}")
    for r in all_layer_rows:
        for l in range(NL):
            slab = row_slab[:, l].copy()
            index = {int(b): i for i, b in enumerate(row_ids)}
            b, s = opaged.locate(batch.block_tables[r], int(batch.positions[r]))
            slab[index[b], 0, :, s, :] = batch.k_new[l, r]
            slab[index[b], 1, :, s, :] = batch.v_new[l, r]
            ref = opaged.decode(Blocks(row_ids, slab), batch.q[l], batch.block_tables, batch.context_lens, SCALE,
                                rows=[r])[0]
            assert_close(got[l, r], ref, f"{batch.name} row {r} layer {l}")
        say(f"  {batch.name} row {r} (context {int(batch.context_lens[r])}): all {NL} layers within tolerance")
    del pool
    torch.cuda.empty_cache()


def test_average_mix_full_pool():
    b = c2_average_mix(seed=1)
    say(f"{b.name}: sum context {int(b.context_lens.sum())}")
    longest = int(np.argmax(b.context_lens))
    _run(b, layers=(0, 31), seed=1001, all_layer_rows=(0, longest))


def test_long_context_full_pool():
    b = c3_long_context(seed=2)
    say(f"{b.name}: 13 x 8192")
    _run(b, layers=(0, 31), seed=1002)
