"""KV append on the GPU against the oracle: bit-exact over the whole pool."""
import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_bits, say, torch_cuda
from workloads import build_batch, c1_tiny

pytestmark = pytest.mark.gpu


def _run_append(batch, layer, torch, q_layer=0):
    pool_d = dev(batch.pool, torch)
    cache = pkv.PagedCache(pool_d)
    pkv.append(cache, layer, dev(batch.k_new[q_layer], torch), dev(batch.v_new[q_layer], torch),
               dev(batch.positions, torch), dev(batch.request_of_token, torch), dev(batch.block_tables, torch))
    torch.cuda.synchronize()
    return host_bits(pool_d)


def test_append_tiny_bitexact():
    torch = torch_cuda()
    b = c1_tiny()
    say(f"append {b.name}")
    got = _run_append(b, 0, torch)
    want = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    assert np.array_equal(got, want)
    # the pinned targets: positions 16, 39, 99, 255 -> logical (block, slot) (1,0), (2,7), (6,3), (15,15)
    for t, (j, s) in enumerate([(1, 0), (2, 7), (6, 3), (15, 15)]):
        blk = b.block_tables[t, j]
        assert np.array_equal(got[blk, 0, 0, :, s, :], b.k_new[0, t])
        assert np.array_equal(got[blk, 0, 1, :, s, :], b.v_new[0, t])


@pytest.mark.parametrize("heads,layers,layer", [(32, 3, 1), (1, 1, 0), (7, 2, 1)])
def test_append_bulk_chunk_bitexact(heads, layers, layer):
    torch = torch_cuda()
    # a 512-token chunk plus three decode rows, multi-layer pool
    b = build_batch("bulk", 21 + heads, [700, 33, 16, 1], [512, 1, 1, 1], num_blocks=80, num_layers=layers,
                    num_heads=heads, stride=48)
    say(f"append bulk heads={heads} layers={layers} layer={layer}")
    got = _run_append(b, layer, torch, q_layer=layer)
    want = opaged.append(b.pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                         b.block_tables)
    assert np.array_equal(got, want)


def test_append_skips_out_of_range_targets():
    torch = torch_cuda()
    b = c1_tiny(seed=5)
    bad_pos = b.positions.copy()
    bad_pos[1] = 16 * 16  # past the table stride -> skipped, nothing else touched
    bad_rows = b.request_of_token.copy()
    bad_rows[2] = 9       # no such row -> skipped
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    pkv.append(cache, 0, dev(b.k_new[0], torch), dev(b.v_new[0], torch), dev(bad_pos, torch), dev(bad_rows, torch),
               dev(b.block_tables, torch))
    torch.cuda.synchronize()
    keep = [0, 3]
    want = opaged.append(b.pool, 0, b.k_new[0][keep], b.v_new[0][keep], b.positions[keep],
                         b.request_of_token[keep], b.block_tables)
    assert np.array_equal(host_bits(pool_d), want)
