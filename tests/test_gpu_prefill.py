"""Chunked-prefill attention (MFMA) mixed with decode rows, on the GPU, against
the fp64 oracle; plus bitwise invariants of the mixed launch."""
import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, ramp_keys, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch, c5_mixed

pytestmark = pytest.mark.gpu


def gpu_prefill(b, torch, *, layer=0, pool=None, append=True):
    pool = b.pool if pool is None else pool
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    tables = dev(b.block_tables, torch)
    if append:
        pkv.append(cache, layer, dev(b.k_new[layer], torch), dev(b.v_new[layer], torch), dev(b.positions, torch),
                   dev(b.request_of_token, torch), tables)
    T = b.total_q
    maxL = int(b.context_lens.max())
    maxq = int(b.q_counts.max())
    ws = torch.empty(pkv.prefill_workspace_size(cache, b.rows, T, maxq, maxL), dtype=torch.uint8, device="cuda")
    out = torch.full((T, b.num_heads, 128), float("nan"), dtype=torch.float16, device="cuda")
    pkv.chunked_prefill_attention(cache, layer, out, dev(b.q[layer], torch), dev(b.query_start, torch), tables,
                                  dev(b.context_lens, torch), maxq, maxL, SCALE, ws)
    torch.cuda.synchronize()
    bits = out.cpu().numpy().view(np.uint16)
    return bits.view(np.float16).astype(np.float64), bits


def oracle_prefill(b, layer=0):
    pool = opaged.append(b.pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                         b.block_tables)
    return opaged.chunked_prefill(pool[:, layer], b.q[layer], b.query_start, b.block_tables, b.context_lens, SCALE)


def _many_rows(n):
    """n rows of seeded lengths in [2, 1500); about a quarter are decode rows (one query), the rest chunks of up to
    300 queries."""
    lens = np.random.default_rng(78).integers(2, 1500, n)
    want = np.random.default_rng(79).integers(-60, 300, n)
    return [int(L) for L in lens], [int(max(1, min(w, L))) for w, L in zip(want, lens)]


CASES = [
    # name, heads, lens, q_counts
    ("chunk-and-decode", 32, [700, 40, 300, 17], [300, 1, 1, 1]),
    ("tile-edges", 32, [129, 130, 256, 2, 1000], [128, 129, 256, 2, 1]),
    ("ranges", 8, [5000, 2100, 4100], [200, 2100, 64]),
    ("odd-heads", 5, [900, 33, 2049], [257, 1, 3]),
    # a decode row of 67 ranges and a chunk of 9 prefill ranges, merged in the same call
    ("long-rows", 2, [17000, 18200, 600], [1, 140, 300]),
    # the most KV heads the pool accepts
    ("max-heads", 128, [300, 40], [70, 1]),
    # more rows than one wave's lanes: the tile search and the decode rows step through rows 64 at a time
    ("many-rows", 4, *_many_rows(150)),
]
# block tables exactly as long as the longest row needs (max_context_len = 16 * bt_stride)
FULL_TABLE = ("full-tables", 8, [2048, 1000, 2047], [256, 1, 2047])


def test_prefill_full_tables():
    torch = torch_cuda()
    name, heads, lens, qc = FULL_TABLE
    b = build_batch(name, 301, lens, qc, num_blocks=sum(-(-L // 16) for L in lens) + 4, num_heads=heads, stride=128)
    assert b.block_tables.shape[1] * 16 == max(lens)
    say(f"prefill {name} lens={lens} q={qc}")
    got, _ = gpu_prefill(b, torch)
    say(f"  {assert_close(got, oracle_prefill(b), name)}")


@pytest.mark.parametrize("name,heads,lens,qc", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(name, heads, lens, qc):
    torch = torch_cuda()
    nb = sum(-(-L // 16) for L in lens)
    b = build_batch(name, 300 + heads, lens, qc, num_blocks=nb + 12, num_heads=heads,
                    stride=max(-(-L // 16) for L in lens) + 2)
    say(f"prefill {name} heads={heads} lens={lens} q={qc}")
    got, _ = gpu_prefill(b, torch)
    s = assert_close(got, oracle_prefill(b), name)
    say(f"  {s}")


def test_prefill_mixed_c5_shape():
    """One 512-token chunk at offset 7,488 of an 8,000-token prompt plus 31
    average-mix decode rows, checked element by element."""
    torch = torch_cuda()
    shape = c5_mixed(with_pool=False)
    used = int(sum(-(-int(L) // 16) for L in shape.context_lens))
    b = c5_mixed(with_pool=True, num_blocks=used + 8, poison=True)
    say(f"prefill {b.name}: {b.rows} rows, {b.total_q} queries, {used} blocks")
    got, _ = gpu_prefill(b, torch)
    s = assert_close(got, oracle_prefill(b), b.name)
    say(f"  {s}")


def test_mixed_decode_rows_equal_decode_launch_bitwise():
    torch = torch_cuda()
    lens = [1500, 40, 2600, 17, 600]
    b = build_batch("mixed-vs-decode", 41, lens, [300, 1, 1, 1, 1], num_blocks=420, stride=170)
    _, mixed = gpu_prefill(b, torch)
    # the decode rows alone, through pkv_decode_attention on the same appended pool
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    pkv.append(cache, 0, dev(b.k_new[0], torch), dev(b.v_new[0], torch), dev(b.positions, torch),
               dev(b.request_of_token, torch), dev(b.block_tables, torch))
    rows = [1, 2, 3, 4]
    tables = dev(np.ascontiguousarray(b.block_tables[rows]), torch)
    lens_d = dev(b.context_lens[rows], torch)
    tok = b.query_start[rows]
    q = dev(np.ascontiguousarray(b.q[0][tok]), torch)
    ws = torch.empty(pkv.decode_workspace_size(cache, 4, 2600), dtype=torch.uint8, device="cuda")
    out = torch.empty((4, 32, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention(cache, 0, out, q, tables, lens_d, 2600, SCALE, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), mixed[tok])


def test_prefill_batch_invariance_bitwise():
    torch = torch_cuda()
    lens = [3000, 700, 90]
    qc = [400, 1, 50]
    b = build_batch("inv", 42, lens, qc, num_blocks=260, stride=200)
    _, full = gpu_prefill(b, torch)
    # row 0 alone
    one = build_batch("one", 0, [lens[0]], [qc[0]], num_blocks=260, stride=200, with_pool=False)
    one.pool = b.pool
    one.block_tables = np.ascontiguousarray(b.block_tables[:1])
    sl = slice(0, qc[0])
    one.k_new, one.v_new, one.q = b.k_new[:, sl].copy(), b.v_new[:, sl].copy(), b.q[:, sl].copy()
    _, alone = gpu_prefill(one, torch)
    assert np.array_equal(alone, full[sl])


def test_chunk_last_query_matches_decode():
    torch = torch_cuda()
    b = build_batch("last", 43, [2500], [256], num_blocks=170, stride=160)
    got, _ = gpu_prefill(b, torch)
    ref = oracle_prefill(b)
    assert_close(got[-1], ref[-1], "last query")
    # the same last query as a decode row over the appended pool
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    dec = opaged.decode(pool[:, 0], b.q[0][-1:], b.block_tables, [2500], SCALE)
    np.testing.assert_allclose(ref[-1], dec[0], rtol=0, atol=1e-12)


def test_split_chunk_matches_one_call():
    torch = torch_cuda()
    # one 384-query chunk vs two 192-query chunks over the same prompt
    b = build_batch("one-call", 44, [4000], [384], num_blocks=260, stride=260)
    got, _ = gpu_prefill(b, torch)
    first = build_batch("first", 0, [4000 - 192], [192], num_blocks=260, stride=260, with_pool=False)
    first.pool, first.block_tables = b.pool, b.block_tables
    first.k_new, first.v_new, first.q = (x[:, :192].copy() for x in (b.k_new, b.v_new, b.q))
    g1, _ = gpu_prefill(first, torch)
    assert_close(g1, got[:192], "first half")
    ref = oracle_prefill(b)
    assert_close(got, ref, "one call")


def test_prefill_growing_scores():
    """Keys grow along the context (up to 8x): a chunk's exponent reference must
    move inside a key range, and a decode row's running maximum with it."""
    torch = torch_cuda()
    lens, qc = [2600, 900, 3000], [300, 1, 2]
    b = ramp_keys(build_batch("ramp", 52, lens, qc, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                              stride=max(-(-L // 16) for L in lens) + 2))
    say(f"prefill growing scores lens={lens} q={qc}")
    got, _ = gpu_prefill(b, torch)
    s = assert_close(got, oracle_prefill(b), "growing scores")
    say(f"  {s}")
