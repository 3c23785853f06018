"""Decode attention on the GPU against the fp64 oracle, plus bitwise invariants.

Every case appends the step's new tokens with the library first (decode reads
its own new token), and the oracle appends the same tokens itself."""
import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_f64, ramp_keys, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch, c1_tiny

pytestmark = pytest.mark.gpu


def gpu_decode(batch, torch, *, pool=None, tables=None, q=None, lens=None, layer=0, append=True):
    pool = batch.pool if pool is None else pool
    tables = batch.block_tables if tables is None else tables
    q = batch.q[layer] if q is None else q
    lens = batch.context_lens if lens is None else lens
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    tables_d = dev(tables, torch)
    if append:
        pkv.append(cache, layer, dev(batch.k_new[layer], torch), dev(batch.v_new[layer], torch),
                   dev(batch.positions, torch), dev(batch.request_of_token, torch), tables_d)
    R = len(lens)
    maxL = int(np.max(lens))
    ws = torch.empty(max(pkv.decode_workspace_size(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, cache.num_heads, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention(cache, layer, out, dev(q, torch), tables_d, dev(np.asarray(lens, np.int32), torch), maxL,
                         SCALE, ws)
    torch.cuda.synchronize()
    return host_f64(out.view(torch.int16)), out.cpu().numpy().view(np.uint16)


def oracle_decode(batch, layer=0):
    pool = opaged.append(batch.pool, layer, batch.k_new[layer], batch.v_new[layer], batch.positions,
                         batch.request_of_token, batch.block_tables)
    return opaged.decode(pool[:, layer], batch.q[layer], batch.block_tables, batch.context_lens, SCALE)


def test_decode_full_tables():
    """Block tables exactly as long as the longest row needs (max_context_len =
    16 * bt_stride): the last table entry is read, and nothing past it."""
    torch = torch_cuda()
    lens = [1024, 16, 1023, 257]
    b = build_batch("full-tables", 33, lens, np.ones(len(lens)), num_blocks=sum(-(-L // 16) for L in lens) + 4,
                    num_layers=1, num_heads=8, stride=64)
    assert b.block_tables.shape[1] * 16 == max(lens)
    say(f"decode with full tables lens={lens}")
    got, _ = gpu_decode(b, torch)
    say(f"  {assert_close(got, oracle_decode(b), 'full tables')}")


def test_decode_tiny():
    torch = torch_cuda()
    b = c1_tiny()
    say(f"decode {b.name}")
    got, _ = gpu_decode(b, torch)
    s = assert_close(got, oracle_decode(b), b.name)
    say(f"  {s}")


CASES = [
    # name, heads, layers, lens
    ("ragged-one-split", 32, 1, [1, 2, 15, 16, 17, 31, 33, 100, 255, 256, 257, 511, 512]),
    ("multi-split", 32, 2, [513, 1000, 1024, 1025, 1537, 2047, 2600]),
    ("odd-heads", 5, 1, [1, 600, 3, 1300]),
    ("one-head-long", 1, 1, [4100, 8192]),
    # more than 64 ranges per row: the merge takes its ranges in several passes of 64
    ("beyond-64-ranges", 2, 1, [20000, 16400, 16385, 7]),
    # the most heads the library accepts (32 workgroups of 4 heads per range)
    ("max-heads", 128, 2, [300, 17, 1]),
    # many rows of mixed lengths (one and several ranges)
    ("many-rows", 4, 1, [int(x) for x in np.random.default_rng(77).integers(1, 900, 700)]),
]


@pytest.mark.parametrize("name,heads,layers,lens", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(name, heads, layers, lens):
    torch = torch_cuda()
    nb = sum(-(-L // 16) for L in lens)
    b = build_batch(name, 100 + heads, lens, np.ones(len(lens)), num_blocks=nb + 20, num_layers=layers,
                    num_heads=heads, stride=max(-(-L // 16) for L in lens) + 3)
    layer = layers - 1
    say(f"decode {name} heads={heads} lens={lens}")
    got, _ = gpu_decode(b, torch, layer=layer)
    s = assert_close(got, oracle_decode(b, layer), name)
    say(f"  {s}")


def _batch(seed=7, lens=(40, 700, 1500, 17, 2100), heads=32, **kw):
    nb = sum(-(-L // 16) for L in lens)
    return build_batch("inv", seed, list(lens), np.ones(len(lens)), num_blocks=nb + 16, num_heads=heads,
                       stride=max(-(-L // 16) for L in lens) + 2, **kw)


def test_block_permutation_invariance_bitwise():
    torch = torch_cuda()
    b = _batch()
    _, base = gpu_decode(b, torch)
    perm = np.random.default_rng(3).permutation(b.num_blocks)
    pool2 = np.empty_like(b.pool)
    pool2[perm] = b.pool
    tables2 = perm[b.block_tables].astype(np.int32)
    _, moved = gpu_decode(b, torch, pool=pool2, tables=tables2)
    assert np.array_equal(base, moved)


def test_batch_invariance_bitwise():
    torch = torch_cuda()
    b = _batch(seed=8)
    _, base = gpu_decode(b, torch)
    for r in range(b.rows):
        # the row alone: its own token appended, its own query, nothing else in the batch
        one = build_batch("x", 0, [int(b.context_lens[r])], [1], num_blocks=b.num_blocks, num_heads=b.num_heads,
                          stride=b.bt_stride, with_pool=False)
        one.pool = b.pool
        one.block_tables = b.block_tables[r:r + 1]
        one.k_new = b.k_new[:, r:r + 1]
        one.v_new = b.v_new[:, r:r + 1]
        one.q = b.q[:, r:r + 1]
        _, alone = gpu_decode(one, torch)
        assert np.array_equal(alone[0], base[r]), r


def test_shared_prefix_matches_private_copies_bitwise():
    torch = torch_cuda()
    lens = [1000, 800, 1200]
    P = 40  # shared full blocks (640 tokens)
    b = build_batch("shared", 9, lens, [1, 1, 1], num_blocks=200, stride=80, shared_prefix_blocks=P,
                    shared_rows=[1, 2])
    _, shared = gpu_decode(b, torch)
    # private copies: rows 1 and 2 get their own copies of the prefix blocks
    pool = b.pool.copy()
    tables = b.block_tables.copy()
    spare = list(b.free_after[::-1])
    for r in (1, 2):
        for j in range(P):
            nid = int(spare.pop())
            pool[nid] = pool[tables[r, j]]
            tables[r, j] = nid
    _, private = gpu_decode(b, torch, pool=pool, tables=tables)
    assert np.array_equal(shared, private)
    assert_close(host := shared.view(np.float16).astype(np.float64), oracle_decode(b), "shared")


def test_marker_constant_values():
    torch = torch_cuda()
    b = _batch(seed=10, lens=(33, 512, 513, 1999))
    consts = np.array([0.625, -1.5, 0.0078125, 3.0], dtype=np.float16)
    pool = b.pool.copy()
    for r, L in enumerate(b.context_lens):
        for j in range(-(-int(L) // 16)):
            blk = b.block_tables[r, j]
            pool[blk, :, 1] = consts[r].view(np.uint16)
    b.v_new = np.broadcast_to(consts.view(np.uint16)[None, :, None, None], b.v_new.shape).copy()
    got, _ = gpu_decode(b, torch, pool=pool)
    for r in range(b.rows):
        assert np.all(got[r] == float(consts[r])), r


def test_poisoned_slots_do_not_leak():
    torch = torch_cuda()
    b = _batch(seed=11, lens=(17, 31, 529, 1041))
    assert np.isnan(b.pool.view(np.float16)).any()
    got, _ = gpu_decode(b, torch)
    assert np.isfinite(got).all()
    assert_close(got, oracle_decode(b), "poison")


def test_decode_growing_scores():
    """Keys grow along the context (up to 8x), so every range's running maximum
    keeps moving and old partial sums are rescaled many times."""
    torch = torch_cuda()
    lens = [300, 1100, 2600, 40]
    b = ramp_keys(build_batch("ramp", 51, lens, np.ones(len(lens)), num_blocks=sum(-(-L // 16) for L in lens) + 8,
                              stride=max(-(-L // 16) for L in lens) + 2))
    say(f"decode growing scores lens={lens}")
    got, _ = gpu_decode(b, torch)
    s = assert_close(got, oracle_decode(b), "growing scores")
    say(f"  {s}")


@pytest.mark.parametrize("heads", [32, 5])
def test_appending_decode_equals_append_then_decode_bitwise(heads):
    """pkv_decode_attention_append leaves the same pool bytes and the same
    output bits as pkv_append followed by pkv_decode_attention, for rows that
    end on, just past and inside block and range boundaries, in the second
    layer of a two-layer pool (5 heads: a workgroup with idle waves)."""
    torch = torch_cuda()
    lens = [1, 16, 17, 255, 256, 257, 700, 2600]
    b = build_batch("fused", 61, lens, np.ones(len(lens)), num_blocks=sum(-(-L // 16) for L in lens) + 6,
                    num_layers=2, num_heads=heads, stride=max(-(-L // 16) for L in lens) + 2)
    layer = 1
    say(f"appending decode vs append + decode, lens={lens}")
    _, ref_bits = gpu_decode(b, torch, layer=layer)
    pool_ref = opaged.append(b.pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                             b.block_tables)
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    R, maxL = len(lens), max(lens)
    ws = torch.empty(pkv.decode_workspace_size(cache, R, maxL), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_append(cache, layer, out, dev(b.q[layer], torch), dev(b.k_new[layer], torch),
                                dev(b.v_new[layer], torch), dev(b.block_tables, torch), dev(b.context_lens, torch),
                                maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert np.array_equal(pool_d.cpu().numpy().view(np.uint16), pool_ref), "fused append differs from pkv_append"
    assert np.array_equal(out.cpu().numpy().view(np.uint16), ref_bits), "fused decode differs from append + decode"
