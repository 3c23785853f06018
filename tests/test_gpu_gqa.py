"""Grouped-query attention on the GPU: G query heads share each KV head of the
pool.  Parity with the oracle; decode batch invariance; and, for prefill,
bitwise equality with multi-head attention over a pool in which every query
head holds a copy of its KV head."""
import numpy as np
import pytest

import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_bits, host_f64, ramp_keys, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch

pytestmark = pytest.mark.gpu


def _full_pool(b):
    """The batch's pool with every layer's new tokens appended (a bit copy; the
    library's append is checked bit for bit against this in its own tests)."""
    pool = b.pool
    for layer in range(pool.shape[1]):
        pool = opaged.append(pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                             b.block_tables)
    return pool


def _queries(seed, T, Hq):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, Hq, 128), dtype=np.float32).astype(np.float16).view(np.uint16)


def _decode(torch, pool, Hq, layer, q, tables, lens):
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    R = len(lens)
    maxL = int(np.max(lens))
    ws = torch.empty(max(pkv.decode_workspace_size_gqa(cache, Hq, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, Hq, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_gqa(cache, Hq, layer, out, dev(q, torch), dev(tables, torch), dev(lens, torch), maxL, SCALE,
                             ws)
    torch.cuda.synchronize()
    return out


def _duplicate_heads(pool, G):
    """The pool with every KV head copied to its G query heads (multi-head layout)."""
    return np.ascontiguousarray(np.repeat(pool, G, axis=3))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_decode_parity(G):
    torch = torch_cuda()
    Hkv = 8 if G < 8 else 4
    Hq = Hkv * G
    # lengths at the edges of a block, of a wave's share of a range (64 tokens
    # on the matrix-core fold, 128 on the vector one) and of a range
    lens = [1, 15, 16, 17, 63, 64, 65, 127, 129, 191, 193, 255, 256, 257, 700, 2600]
    b = build_batch(f"gqa-decode-G{G}", 40 + G, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=2, num_heads=Hkv, stride=170)
    q = _queries(50 + G, len(lens), Hq)
    pool = _full_pool(b)
    say(f"gqa decode G={G} Hkv={Hkv}")
    for layer in (0, 1):
        got = _decode(torch, pool, Hq, layer, q, b.block_tables, b.context_lens)
        ref = opaged.decode(pool[:, layer], q, b.block_tables, b.context_lens, SCALE, group=G)
        assert_close(host_f64(got), ref, f"G={G} layer {layer}")


def test_gqa_decode_odd_kv_heads():
    """3 KV heads of 4 query heads each: 12 query heads, a merge grid of three
    4-head groups."""
    torch = torch_cuda()
    G, Hkv = 4, 3
    Hq = Hkv * G
    lens = [1, 17, 256, 257, 1300]
    b = build_batch("gqa-odd", 47, lens, [1] * len(lens), num_blocks=130, num_layers=1, num_heads=Hkv, stride=90)
    q = _queries(57, len(lens), Hq)
    pool = _full_pool(b)
    say(f"gqa decode G={G} Hkv={Hkv}")
    got = _decode(torch, pool, Hq, 0, q, b.block_tables, b.context_lens)
    ref = opaged.decode(pool[:, 0], q, b.block_tables, b.context_lens, SCALE, group=G)
    assert_close(host_f64(got), ref, f"G={G} Hkv={Hkv}")


def test_gqa_decode_many_rows():
    """500 rows of mixed lengths, 2 KV heads of 4 query heads each."""
    torch = torch_cuda()
    G, Hkv = 4, 2
    lens = [int(x) for x in np.random.default_rng(82).integers(1, 900, 500)]
    b = build_batch("gqa-many", 48, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 4,
                    num_heads=Hkv, stride=max(-(-L // 16) for L in lens))
    q = _queries(49, len(lens), Hkv * G)
    pool = _full_pool(b)
    say(f"gqa decode many rows: {len(lens)}")
    got = _decode(torch, pool, Hkv * G, 0, q, b.block_tables, b.context_lens)
    ref = opaged.decode(pool[:, 0], q, b.block_tables, b.context_lens, SCALE, group=G)
    assert_close(host_f64(got), ref, "gqa many rows")


def test_gqa_decode_beyond_64_ranges():
    """Grouped decode (G = 4) over rows of 79 and 65 ranges: the merge takes its
    ranges in several passes of 64."""
    torch = torch_cuda()
    G, Hkv = 4, 2
    lens = [20000, 16400, 90]
    b = build_batch("gqa-long", 44, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 4,
                    num_heads=Hkv, stride=max(-(-L // 16) for L in lens))
    q = _queries(45, len(lens), Hkv * G)
    pool = _full_pool(b)
    say(f"gqa decode beyond 64 ranges lens={lens}")
    got = _decode(torch, pool, Hkv * G, 0, q, b.block_tables, b.context_lens)
    ref = opaged.decode(pool[:, 0], q, b.block_tables, b.context_lens, SCALE, group=G)
    assert_close(host_f64(got), ref, "gqa beyond 64 ranges")


@pytest.mark.parametrize("G", [4, 8])
def test_gqa_decode_growing_scores(G):
    """Keys grow along the context (up to 8x), so the grouped fold's deferred
    exponent reference moves again and again inside a range."""
    torch = torch_cuda()
    Hkv = 8 if G < 8 else 4
    Hq = Hkv * G
    lens = [300, 1100, 2600, 40]
    b = ramp_keys(build_batch(f"gqa-ramp-G{G}", 60 + G, lens, [1] * len(lens),
                              num_blocks=sum(-(-L // 16) for L in lens) + 8, num_heads=Hkv, stride=170))
    q = _queries(70 + G, len(lens), Hq)
    pool = _full_pool(b)
    say(f"gqa decode growing scores G={G}")
    got = _decode(torch, pool, Hq, 0, q, b.block_tables, b.context_lens)
    ref = opaged.decode(pool[:, 0], q, b.block_tables, b.context_lens, SCALE, group=G)
    assert_close(host_f64(got), ref, f"growing scores G={G}")


@pytest.mark.parametrize("G", [2, 4, 8])
def test_gqa_decode_batch_invariance_bitwise(G):
    """A row's grouped-query output does not depend on its batch neighbours:
    each row decoded alone gives the same bits as inside the batch."""
    torch = torch_cuda()
    Hkv = 4
    Hq = Hkv * G
    lens = [40, 300, 1100, 4100]
    b = build_batch(f"gqa-inv-G{G}", 60 + G, lens, [1] * len(lens), num_blocks=400, num_layers=1, num_heads=Hkv,
                    stride=260)
    q = _queries(70 + G, len(lens), Hq)
    pool = _full_pool(b)
    say(f"gqa decode batch invariance G={G}")
    full = host_bits(_decode(torch, pool, Hq, 0, q, b.block_tables, b.context_lens))
    for r in range(len(lens)):
        alone = host_bits(_decode(torch, pool, Hq, 0, q[r:r + 1], b.block_tables[r:r + 1], b.context_lens[r:r + 1]))
        assert np.array_equal(alone[0], full[r])


def _prefill(torch, pool, Hq, q, b):
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    T = int(b.total_q)
    maxq = int(b.q_counts.max())
    maxL = int(b.context_lens.max())
    ws = torch.empty(pkv.prefill_workspace_size_gqa(cache, Hq, b.rows, T, maxq, maxL), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((T, Hq, 128), dtype=torch.float16, device="cuda")
    pkv.chunked_prefill_attention_gqa(cache, Hq, 0, out, dev(q, torch), dev(b.query_start, torch),
                                      dev(b.block_tables, torch), dev(b.context_lens, torch), maxq, maxL, SCALE, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_prefill_parity_and_duplicated_heads(G):
    torch = torch_cuda()
    Hkv = 8
    Hq = Hkv * G
    b = build_batch(f"gqa-prefill-G{G}", 80 + G, [2300, 700, 40], [300, 1, 1], num_blocks=220, num_layers=1,
                    num_heads=Hkv, stride=150)
    q = _queries(90 + G, int(b.total_q), Hq)
    pool = _full_pool(b)
    say(f"gqa prefill G={G}")
    got = _prefill(torch, pool, Hq, q, b)
    ref = opaged.chunked_prefill(pool[:, 0], q, b.query_start, b.block_tables, b.context_lens, SCALE, group=G)
    assert_close(host_f64(got), ref, f"prefill G={G}")
    want = _prefill(torch, _duplicate_heads(pool, G), Hq, q, b)
    assert np.array_equal(host_bits(got), host_bits(want))


@pytest.mark.parametrize("G", [2, 4, 8])
def test_gqa_appending_decode_equals_append_then_decode_bitwise(G):
    """pkv_decode_attention_append_gqa leaves the same pool bytes and output
    bits as pkv_append followed by pkv_decode_attention_gqa."""
    torch = torch_cuda()
    Hkv = 8 if G < 8 else 4
    Hq = Hkv * G
    lens = [1, 16, 17, 63, 64, 65, 257, 700, 2600]
    b = build_batch(f"gqa-fused-G{G}", 80 + G, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 6,
                    num_layers=2, num_heads=Hkv, stride=max(-(-L // 16) for L in lens) + 2)
    q = _queries(90 + G, len(lens), Hq)
    layer = 1
    R, maxL = len(lens), max(lens)
    say(f"gqa appending decode G={G} vs append + decode")

    def run(fused):
        pool_d = dev(b.pool, torch)
        cache = pkv.PagedCache(pool_d)
        ws = torch.empty(pkv.decode_workspace_size_gqa(cache, Hq, R, maxL), dtype=torch.uint8, device="cuda")
        out = torch.empty((R, Hq, 128), dtype=torch.float16, device="cuda")
        tables, lens_d = dev(b.block_tables, torch), dev(b.context_lens, torch)
        k, v = dev(b.k_new[layer], torch), dev(b.v_new[layer], torch)
        if fused:
            pkv.decode_attention_append_gqa(cache, Hq, layer, out, dev(q, torch), k, v, tables, lens_d, maxL, SCALE, ws)
        else:
            pkv.append(cache, layer, k, v, dev(b.positions, torch), dev(b.request_of_token, torch), tables)
            pkv.decode_attention_gqa(cache, Hq, layer, out, dev(q, torch), tables, lens_d, maxL, SCALE, ws)
        torch.cuda.synchronize()
        return pool_d.cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16)

    pool_a, out_a = run(False)
    pool_b, out_b = run(True)
    assert np.array_equal(pool_a, pool_b), "fused append differs from pkv_append"
    assert np.array_equal(out_a, out_b), "fused grouped decode differs from append + decode"
