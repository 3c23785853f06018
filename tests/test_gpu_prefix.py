"""Shared-prefix decode on the GPU: rows that share a ref-counted prefix of P
blocks read it once per step through matrix-core tiles; the result must still
be every row's attention over its own context.

Parity with the oracle's plain decode (R8 tolerance) for aligned and ragged
prefixes, one to three tiles of sharing rows, and several layers; bitwise
checks that rows without the mark, and a prefix of zero blocks, give exactly
the plain decode's bits, and that a sharing row's output does not depend on
the rest of the batch."""
import zlib

import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_bits, host_f64, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch

pytestmark = pytest.mark.gpu


def _full_pool(b):
    pool = b.pool
    for layer in range(pool.shape[1]):
        pool = opaged.append(pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                             b.block_tables)
    return pool


def _prefix(torch, pool_d, layer, q, tables, lens, marks, P):
    cache = pkv.PagedCache(pool_d)
    R = len(lens)
    maxL = int(np.max(lens))
    ws = torch.empty(max(pkv.decode_workspace_size_prefix(cache, R, maxL, P), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, cache.num_heads, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_prefix(cache, layer, out, dev(q, torch), dev(tables, torch), dev(lens, torch), maxL, SCALE,
                                dev(np.asarray(marks, dtype=np.int32), torch), P, ws)
    torch.cuda.synchronize()
    return out


def _plain(torch, pool_d, layer, q, tables, lens):
    cache = pkv.PagedCache(pool_d)
    R = len(lens)
    maxL = int(np.max(lens))
    ws = torch.empty(max(pkv.decode_workspace_size(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, cache.num_heads, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention(cache, layer, out, dev(q, torch), dev(tables, torch), dev(lens, torch), maxL, SCALE, ws)
    torch.cuda.synchronize()
    return out


def _case(name):
    """(batch, marks, P).  Row 0 owns the prefix; rows in `shared` point their
    first P table entries at it and are marked.  `lone` rows are marked but
    end inside the prefix length, with private tables: they must be decoded
    like unmarked rows."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "ragged-125":      # the 2,000-token prefix: 7 full ranges and one of 13 blocks
        P, layers, H = 125, 1, 32
        lens = [2300] + list(rng.integers(2001, 5001, 29)) + list(rng.integers(1, 3001, 10))
        shared = range(1, 30)
        lone = []
    elif name == "aligned-3-tiles":  # 70 sharing rows: three tiles of 32
        P, layers, H = 16, 1, 8
        lens = [1100, 257, 272] + list(rng.integers(257, 1101, 67)) + [40, 700, 256, 3, 1500]
        shared = range(1, 70)
        lone = [72]                # L = 256 = 16 P
    elif name == "one-block":
        P, layers, H = 1, 1, 32
        lens = [40, 17, 300, 33, 16, 5, 2000]
        shared = [1, 2, 3, 6]
        lone = [4]                 # L = 16 = 16 P
    elif name == "heads-12":        # a suffix workgroup of 8 heads with only 4 in use
        P, layers, H = 20, 1, 12
        lens = [400, 350, 800, 330, 20, 1500, 321]
        shared = [1, 2, 3, 5, 6]
        lone = []
    elif name == "odd-37-two-layers":
        P, layers, H = 37, 2, 32
        lens = [600, 593, 1000, 4000, 40, 2600, 900, 1200, 600, 601, 3000, 7]
        shared = [1, 2, 3, 5, 6, 7, 8, 9, 10]
        lone = []
    else:
        raise KeyError(name)
    R = len(lens)
    nblk = [-(-int(L) // 16) for L in lens]
    need = sum(nblk) - len(list(shared)) * P + 8
    b = build_batch(f"prefix-{name}", 7, lens, [1] * R, num_blocks=need, num_layers=layers, num_heads=H,
                    stride=max(nblk), shared_prefix_blocks=P, shared_rows=shared)
    marks = np.zeros(R, dtype=np.int32)
    marks[0] = 1
    marks[list(shared)] = 1
    marks[list(lone)] = 1
    return b, marks, P


CASES = ["ragged-125", "aligned-3-tiles", "one-block", "heads-12", "odd-37-two-layers"]


@pytest.mark.parametrize("name", CASES)
def test_prefix_decode_parity(name):
    torch = torch_cuda()
    b, marks, P = _case(name)
    pool = _full_pool(b)
    pool_d = dev(pool, torch)
    for layer in range(b.num_layers):
        say(f"prefix decode {name} P={P} layer {layer} rows={b.rows} marked={int(marks.sum())}")
        got = _prefix(torch, pool_d, layer, b.q[layer], b.block_tables, b.context_lens, marks, P)
        ref = opaged.decode(pool[:, layer], b.q[layer], b.block_tables, b.context_lens, SCALE)
        assert_close(host_f64(got), ref, f"{name} layer {layer}")
        # rows that do not take the shared path give the plain decode's bits
        plain = host_bits(_plain(torch, pool_d, layer, b.q[layer], b.block_tables, b.context_lens))
        bits = host_bits(got)
        for r in range(b.rows):
            if not (marks[r] and b.context_lens[r] > 16 * P):
                assert np.array_equal(bits[r], plain[r]), (name, layer, r)


def test_prefix_of_zero_blocks_is_plain_decode():
    torch = torch_cuda()
    b, marks, _ = _case("odd-37-two-layers")
    pool = _full_pool(b)
    pool_d = dev(pool, torch)
    say("prefix decode with P = 0")
    got = host_bits(_prefix(torch, pool_d, 1, b.q[1], b.block_tables, b.context_lens, marks, 0))
    want = host_bits(_plain(torch, pool_d, 1, b.q[1], b.block_tables, b.context_lens))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["ragged-125", "aligned-3-tiles"])
def test_prefix_decode_batch_invariance_bitwise(name):
    """A sharing row's bits do not depend on which other rows share its tile:
    decoded alone (with its mark, over the same pool) it gives the same bits."""
    torch = torch_cuda()
    b, marks, P = _case(name)
    pool = _full_pool(b)
    pool_d = dev(pool, torch)
    say(f"prefix decode batch invariance {name}")
    full = host_bits(_prefix(torch, pool_d, 0, b.q[0], b.block_tables, b.context_lens, marks, P))
    for r in (0, 1, 2, b.rows - 1, 40):
        if r >= b.rows:
            continue
        alone = _prefix(torch, pool_d, 0, b.q[0][r:r + 1], b.block_tables[r:r + 1], b.context_lens[r:r + 1],
                        marks[r:r + 1], P)
        assert np.array_equal(host_bits(alone)[0], full[r]), (name, r)
