"""Whole-block copies on the GPU (copy-on-write and swap) against the oracle:
bit-exact over the whole pool and the whole host image."""
import numpy as np
import pytest

import oracle.blocks as oblocks
import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_bits, host_f64, say, torch_cuda
from tests.tolerance import assert_close

pytestmark = pytest.mark.gpu


def _rand_pool(seed, shape):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("layers,heads", [(3, 5), (2, 32), (32, 32)])
def test_copy_blocks_bitexact(layers, heads):
    torch = torch_cuda()
    nb = 12 if layers == 32 else 40
    pool = _rand_pool(100 + layers, (nb, layers, 2, heads, 16, 128))
    # distinct destinations that are not sources; one pair with an id outside the pool is skipped
    src = np.array([1, 7, nb - 2, 3, nb + 5], dtype=np.int32)
    dst = np.array([nb - 1, 2, 0, 5, 4], dtype=np.int32)
    say(f"copy_blocks layers={layers} heads={heads} block={layers * 2 * heads * 4} KiB")
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    assert pkv.block_bytes(cache) == layers * 2 * heads * 16 * 128 * 2
    pkv.copy_blocks(cache, dev(src, torch), dev(dst, torch))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(pool_d), oblocks.copy_blocks(pool, src, dst))


def test_swap_roundtrip_bitexact():
    torch = torch_cuda()
    layers, heads, nb = 2, 32, 24
    pool = _rand_pool(7, (nb, layers, 2, heads, 16, 128))
    ids = [5, 6, 7, 20, 3]  # one run of three consecutive ids, two single blocks
    new_ids = [10, 11, 0, 1, 2]
    say("swap out / in")
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    bb = pkv.block_bytes(cache)
    host = torch.empty(len(ids) * bb, dtype=torch.uint8, pin_memory=True)
    pkv.swap_out(cache, ids, host)
    torch.cuda.synchronize()
    image = host.numpy().view(np.uint16).reshape(len(ids), layers, 2, heads, 16, 128)
    assert np.array_equal(image, oblocks.swap_out(pool, ids))
    # the swapped-out blocks' ids are reused: poison their targets, then restore elsewhere
    pool_d[new_ids] = 0x7E00
    pkv.swap_in(cache, host, new_ids)
    torch.cuda.synchronize()
    poisoned = pool.copy()
    poisoned[new_ids] = np.uint16(0x7E00)
    assert np.array_equal(host_bits(pool_d), oblocks.swap_in(poisoned, image, new_ids))


def test_copy_on_write_divergence_decode():
    """Two rows share a 20-token prefix (a full and a partial block).  Row 1
    copies the partial block and appends its own token 20 into the copy; row 0
    appends into the original.  The pool matches the oracle bit for bit and
    both rows' attention matches the oracle."""
    torch = torch_cuda()
    layers, heads, nb = 2, 32, 16
    rng = np.random.default_rng(31)
    pool = _rand_pool(30, (nb, layers, 2, heads, 16, 128))
    full_blk, part_blk, copy_blk = 4, 9, 13
    tables = np.array([[full_blk, part_blk], [full_blk, copy_blk]], dtype=np.int32)
    k_new = rng.standard_normal((layers, 2, heads, 128), dtype=np.float32).astype(np.float16).view(np.uint16)
    v_new = rng.standard_normal((layers, 2, heads, 128), dtype=np.float32).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((2, heads, 128), dtype=np.float32).astype(np.float16).view(np.uint16)
    say("copy-on-write divergence")
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    pkv.copy_blocks(cache, dev(np.array([part_blk], np.int32), torch), dev(np.array([copy_blk], np.int32), torch))
    want = oblocks.copy_blocks(pool, [part_blk], [copy_blk])
    pos = np.array([20, 20], np.int32)
    rot = np.array([0, 1], np.int32)
    tab_d = dev(tables, torch)
    for l in range(layers):
        pkv.append(cache, l, dev(k_new[l], torch), dev(v_new[l], torch), dev(pos, torch), dev(rot, torch), tab_d)
        want = opaged.append(want, l, k_new[l], v_new[l], pos, rot, tables)
    lens = np.array([21, 21], np.int32)
    out = torch.empty((2, heads, 128), dtype=torch.float16, device="cuda")
    for l in range(layers):
        pkv.decode_attention(cache, l, out, dev(q, torch), tab_d, dev(lens, torch), 32, 1.0 / np.sqrt(128.0))
        torch.cuda.synchronize()
        assert_close(host_f64(out), opaged.decode(want[:, l], q, tables, lens, 1.0 / np.sqrt(128.0)), f"layer {l}")
    assert np.array_equal(host_bits(pool_d), want)
