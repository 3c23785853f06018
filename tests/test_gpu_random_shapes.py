"""Decode and chunked prefill at many seeded shapes against the fp64 oracle.

The other GPU tests pick their shapes by hand (edges of blocks, shares and
ranges; many rows; long rows).  Here a seeded draw adds shapes nobody chose:
KV heads in {1, 2, 3, 8}, 1, 2, 4 or 8 query heads per KV head, 1 to 23 rows
of lognormal lengths up to 4,000 tokens, with and without the step's append
fused in (FP16, grouped-query and 8-bit caches), prefill batches that mix
chunks of 2 to 300 queries with decode rows, and shared-prefix decode batches
(prefixes of 1 to 47 blocks, sharing, unmarked and marked-but-short rows),
FP16 and 8-bit appends of flat token lists of up to 300 tokens per row
(bit-exact over the whole pool), and block copies and swaps of seeded id
lists (bit-exact over the pool and the host image).
Each case checks every output element within the tolerance; the fused cases
also check the pool bytes against the oracle's append, and the prefix cases
that rows off the shared path give the plain decode's bits."""
import numpy as np
import pytest

import oracle.blocks as oblocks
import oracle.fp8 as ofp8
import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_f64, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch

pytestmark = pytest.mark.gpu


def _lengths(rng, rows):
    return np.clip(rng.lognormal(5.5, 1.2, rows).astype(np.int64), 1, 4000).tolist()


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 3, 8]))
        group = int(rng.choice([1, 2, 4, 8]))
        lens = _lengths(rng, int(rng.integers(1, 24)))
        out.append((i, hkv, group, lens, bool(rng.integers(0, 2))))
    return out


CASES = _shapes(2024, 24)


@pytest.mark.parametrize("idx,hkv,group,lens,fused", CASES,
                         ids=[f"{c[0]}-kv{c[1]}-g{c[2]}-r{len(c[3])}-{'fused' if c[4] else 'plain'}" for c in CASES])
def test_decode_random_shape(idx, hkv, group, lens, fused):
    torch = torch_cuda()
    hq = hkv * group
    R, maxL = len(lens), max(lens)
    b = build_batch(f"rand-{idx}", 700 + idx, lens, [1] * R, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=2, num_heads=hkv, stride=-(-maxL // 16) + 1)
    layer = 1
    q = np.random.default_rng(900 + idx).standard_normal((R, hq, 128), dtype=np.float32).astype(np.float16)
    q = q.view(np.uint16)
    want_pool = opaged.append(b.pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                              b.block_tables)
    ref = opaged.decode(want_pool[:, layer], q, b.block_tables, b.context_lens, SCALE, group=group)
    pool_d = dev(b.pool if fused else want_pool, torch)
    cache = pkv.PagedCache(pool_d)
    ws = torch.empty(max(pkv.decode_workspace_size_gqa(cache, hq, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, hq, 128), dtype=torch.float16, device="cuda")
    tables, lens_d = dev(b.block_tables, torch), dev(b.context_lens, torch)
    say(f"random decode shape {idx}: {hkv} KV heads, G {group}, {R} rows, longest {maxL}, fused {fused}")
    if fused:
        pkv.decode_attention_append_gqa(cache, hq, layer, out, dev(q, torch), dev(b.k_new[layer], torch),
                                        dev(b.v_new[layer], torch), tables, lens_d, maxL, SCALE, ws)
    else:
        pkv.decode_attention_gqa(cache, hq, layer, out, dev(q, torch), tables, lens_d, maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref, f"random shape {idx}")
    if fused:
        assert np.array_equal(pool_d.cpu().numpy().view(np.uint16), want_pool), "fused append differs"


FP8_CASES = [(i, int(h), _lengths(np.random.default_rng(3000 + i), int(r)))
             for i, (h, r) in enumerate(zip(np.random.default_rng(2025).choice([1, 3, 8, 32], 10),
                                            np.random.default_rng(2026).integers(1, 24, 10)))]


@pytest.mark.parametrize("idx,heads,lens", FP8_CASES, ids=[f"{c[0]}-h{c[1]}-r{len(c[2])}" for c in FP8_CASES])
def test_fp8_decode_random_shape(idx, heads, lens):
    torch = torch_cuda()
    R, maxL = len(lens), max(lens)
    b = build_batch(f"rand8-{idx}", 800 + idx, lens, [1] * R, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=1, num_heads=heads, stride=-(-maxL // 16) + 1)
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    codes, scales = ofp8.quantize_rows(pool)
    ref = ofp8.decode(codes, scales, 0, b.q[0], b.block_tables, b.context_lens, SCALE)
    cache = pkv.PagedCache8(dev(codes, torch), dev(scales, torch))
    ws = torch.empty(max(pkv.decode_workspace_size_fp8(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
    say(f"random 8-bit decode shape {idx}: {heads} heads, {R} rows, longest {maxL}")
    pkv.decode_attention_fp8(cache, 0, out, dev(b.q[0], torch), dev(b.block_tables, torch), dev(b.context_lens, torch),
                             maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref, f"random 8-bit shape {idx}")


def _prefill_shapes(seed, n):
    """KV heads, group size, and rows of lognormal lengths whose query counts
    are 1 (a decode row, about 3 in 10) or a chunk of 2 to 300 queries."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        group = int(rng.choice([1, 2, 4]))
        lens = [max(2, L) for L in _lengths(rng, int(rng.integers(1, 13)))]
        qc = [1 if rng.random() < 0.3 else int(rng.integers(2, min(L, 300) + 1)) for L in lens]
        out.append((i, hkv, group, lens, qc))
    return out


PREFILL_CASES = _prefill_shapes(2027, 8)


@pytest.mark.parametrize("idx,hkv,group,lens,qc", PREFILL_CASES,
                         ids=[f"{c[0]}-kv{c[1]}-g{c[2]}-r{len(c[3])}" for c in PREFILL_CASES])
def test_prefill_random_shape(idx, hkv, group, lens, qc):
    torch = torch_cuda()
    hq = hkv * group
    R, maxL, maxq = len(lens), max(lens), max(qc)
    b = build_batch(f"randp-{idx}", 1100 + idx, lens, qc, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=1, num_heads=hkv, stride=-(-maxL // 16) + 1)
    T = b.total_q
    q = np.random.default_rng(1200 + idx).standard_normal((T, hq, 128), dtype=np.float32).astype(np.float16)
    q = q.view(np.uint16)
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    ref = opaged.chunked_prefill(pool[:, 0], q, b.query_start, b.block_tables, b.context_lens, SCALE, group=group)
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    tables = dev(b.block_tables, torch)
    pkv.append(cache, 0, dev(b.k_new[0], torch), dev(b.v_new[0], torch), dev(b.positions, torch),
               dev(b.request_of_token, torch), tables)
    ws = torch.empty(pkv.prefill_workspace_size_gqa(cache, hq, R, T, maxq, maxL), dtype=torch.uint8, device="cuda")
    out = torch.full((T, hq, 128), float("nan"), dtype=torch.float16, device="cuda")
    say(f"random prefill shape {idx}: {hkv} KV heads, G {group}, {R} rows, {T} queries, longest {maxL}")
    pkv.chunked_prefill_attention_gqa(cache, hq, 0, out, dev(q, torch), dev(b.query_start, torch), tables,
                                      dev(b.context_lens, torch), maxq, maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref, f"random prefill shape {idx}")


def _prefix_shapes(seed, n):
    """(idx, P, heads, lens, shared rows, lone rows): row 0 holds a prefix of P
    blocks that the shared rows reference; lone rows are marked but end inside
    the prefix's length (private tables), the rest are unmarked."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        P = int(rng.integers(1, 48))
        heads = int(rng.choice([8, 32]))
        rows = int(rng.integers(2, 48))
        lens, shared, lone = [], [], []
        for r in range(rows):
            kind = 0 if r == 0 else int(rng.choice(3, p=[0.6, 0.25, 0.15]))
            if kind == 0:
                lens.append(16 * P + 1 + int(min(rng.lognormal(5.0, 1.2), 3000)))
                if r:
                    shared.append(r)
            elif kind == 1:
                lens.append(int(np.clip(rng.lognormal(6.0, 1.2), 1, 5000)))
            else:
                lens.append(int(rng.integers(1, 16 * P + 1)))
                lone.append(r)
        out.append((i, P, heads, lens, shared, lone))
    return out


PREFIX_CASES = _prefix_shapes(2031, 8)


@pytest.mark.parametrize("idx,P,heads,lens,shared,lone", PREFIX_CASES,
                         ids=[f"{c[0]}-P{c[1]}-h{c[2]}-r{len(c[3])}-s{len(c[4])}" for c in PREFIX_CASES])
def test_prefix_decode_random_shape(idx, P, heads, lens, shared, lone):
    torch = torch_cuda()
    R = len(lens)
    nblk = [-(-L // 16) for L in lens]
    say(f"random prefix decode {idx}: P={P}, {heads} heads, {R} rows ({len(shared)} sharing, {len(lone)} lone), "
        f"lengths {min(lens)}..{max(lens)}")
    b = build_batch(f"rand-prefix-{idx}", 1300 + idx, lens, [1] * R, num_blocks=sum(nblk) - len(shared) * P + 8,
                    num_heads=heads, stride=max(nblk), shared_prefix_blocks=P, shared_rows=shared)
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    ref = opaged.decode(pool[:, 0], b.q[0], b.block_tables, b.context_lens, SCALE)
    marks = np.zeros(R, dtype=np.int32)
    marks[[0, *shared, *lone]] = 1
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    maxL = max(lens)
    tables, lens_d, q = dev(b.block_tables, torch), dev(b.context_lens, torch), dev(b.q[0], torch)
    ws = torch.empty(max(pkv.decode_workspace_size_prefix(cache, R, maxL, P), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_prefix(cache, 0, out, q, tables, lens_d, maxL, SCALE, dev(marks, torch), P, ws)
    ws2 = torch.empty(max(pkv.decode_workspace_size(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    plain = torch.empty_like(out)
    pkv.decode_attention(cache, 0, plain, q, tables, lens_d, maxL, SCALE, ws2)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref, f"random prefix decode {idx}")
    # rows that do not take the shared path (unmarked, or ending inside the prefix) give the plain decode's bits
    got, want = out.cpu().numpy().view(np.uint16), plain.cpu().numpy().view(np.uint16)
    for r in range(R):
        if not (marks[r] and lens[r] > 16 * P):
            assert np.array_equal(got[r], want[r]), (idx, r)


def _append_shapes(seed, n):
    """(idx, heads, layers, layer, lens, new-token counts): rows gaining 1 to
    300 tokens at once, over pools of 1 to 3 layers."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        heads = int(rng.choice([1, 3, 8, 32]))
        layers = int(rng.integers(1, 4))
        rows = int(rng.integers(1, 20))
        lens = _lengths(rng, rows)
        counts = [int(min(L, rng.choice([1, 1, int(rng.integers(1, 301))]))) for L in lens]
        out.append((i, heads, layers, int(rng.integers(0, layers)), lens, counts))
    return out


APPEND_CASES = _append_shapes(2033, 10)


@pytest.mark.parametrize("idx,heads,layers,layer,lens,counts", APPEND_CASES,
                         ids=[f"{c[0]}-h{c[1]}-l{c[2]}-r{len(c[4])}-t{sum(c[5])}" for c in APPEND_CASES])
def test_append_random_shape(idx, heads, layers, layer, lens, counts):
    """FP16 and 8-bit appends of a seeded flat token list, bit-exact over the
    whole pool (codes and scales for the 8-bit cache)."""
    torch = torch_cuda()
    R = len(lens)
    b = build_batch(f"rand-append-{idx}", 1400 + idx, lens, counts, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=layers, num_heads=heads, stride=-(-max(lens) // 16) + 1)
    say(f"random append {idx}: {heads} heads, {layers} layers (layer {layer}), {R} rows, {sum(counts)} tokens")
    want = opaged.append(b.pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                         b.block_tables)
    pos, rows, tables = dev(b.positions, torch), dev(b.request_of_token, torch), dev(b.block_tables, torch)
    k, v = dev(b.k_new[layer], torch), dev(b.v_new[layer], torch)
    pool_d = dev(b.pool, torch)
    pkv.append(pkv.PagedCache(pool_d), layer, k, v, pos, rows, tables)
    # the 8-bit cache: every row of the pool quantized, then the same tokens appended
    codes, scales = ofp8.quantize_rows(b.pool)
    want_c, want_s = ofp8.append(codes, scales, layer, b.k_new[layer], b.v_new[layer], b.positions,
                                 b.request_of_token, b.block_tables)
    codes_d, scales_d = dev(codes, torch), dev(scales, torch)
    pkv.append_fp8(pkv.PagedCache8(codes_d, scales_d), layer, k, v, pos, rows, tables)
    torch.cuda.synchronize()
    assert np.array_equal(pool_d.cpu().numpy().view(np.uint16), want)
    assert np.array_equal(codes_d.cpu().numpy(), want_c)
    assert np.array_equal(scales_d.cpu().numpy().view(np.uint32), np.asarray(want_s).view(np.uint32))


COPY_CASES = [(i, int(layers), int(heads)) for i, (layers, heads) in
              enumerate(zip(np.random.default_rng(2035).choice([1, 2, 3, 8], 6),
                            np.random.default_rng(2036).choice([1, 5, 8, 32], 6)))]


@pytest.mark.parametrize("idx,layers,heads", COPY_CASES, ids=[f"{c[0]}-l{c[1]}-h{c[2]}" for c in COPY_CASES])
def test_block_copies_random_shape(idx, layers, heads):
    """Copy-on-write of a seeded set of pairs (distinct destinations, none a
    source; some ids outside the pool, which are skipped), then a swap out and
    back in of seeded id lists: the whole pool and host image bit-exact."""
    torch = torch_cuda()
    rng = np.random.default_rng(1500 + idx)
    nb = int(rng.integers(8, 80))
    pool = rng.standard_normal((nb, layers, 2, heads, 16, 128), dtype=np.float32).astype(np.float16).view(np.uint16)
    perm = rng.permutation(nb)
    n = int(rng.integers(0, nb // 2 + 1))
    src, dst = perm[:n].astype(np.int32), perm[n:2 * n].astype(np.int32)
    if n:
        src[rng.integers(n)] = nb + int(rng.integers(0, 5))   # skipped pair
        dst[rng.integers(n)] = -1 - int(rng.integers(0, 5))   # skipped pair
    say(f"random block copies {idx}: {nb} blocks of {layers} layers x {heads} heads, {n} pairs")
    pool_d = dev(pool, torch)
    cache = pkv.PagedCache(pool_d)
    pkv.copy_blocks(cache, dev(src, torch), dev(dst, torch))
    torch.cuda.synchronize()
    want = oblocks.copy_blocks(pool, src, dst)
    assert np.array_equal(pool_d.cpu().numpy().view(np.uint16), want)
    # swap out a seeded id list (runs of consecutive ids and single ids), then in to other ids
    ids = np.sort(rng.choice(nb, size=int(rng.integers(1, nb // 2 + 1)), replace=False)).tolist()
    back = rng.permutation(nb)[:len(ids)].tolist()
    bb = pkv.block_bytes(cache)
    host = torch.empty(len(ids) * bb, dtype=torch.uint8, pin_memory=True)
    pkv.swap_out(cache, ids, host)
    torch.cuda.synchronize()
    image = host.numpy().view(np.uint16).reshape(len(ids), layers, 2, heads, 16, 128)
    assert np.array_equal(image, oblocks.swap_out(want, ids))
    pkv.swap_in(cache, host, back)
    torch.cuda.synchronize()
    assert np.array_equal(pool_d.cpu().numpy().view(np.uint16), oblocks.swap_in(want, image, back))


FP8_FUSED_CASES = [(i, int(h), _lengths(np.random.default_rng(3100 + i), int(r)))
                   for i, (h, r) in enumerate(zip(np.random.default_rng(2037).choice([1, 3, 8, 32], 6),
                                                  np.random.default_rng(2038).integers(1, 24, 6)))]


@pytest.mark.parametrize("idx,heads,lens", FP8_FUSED_CASES,
                         ids=[f"{c[0]}-h{c[1]}-r{len(c[2])}" for c in FP8_FUSED_CASES])
def test_fp8_fused_append_decode_random_shape(idx, heads, lens):
    """The 8-bit decode with the step's append fused in: codes and scales
    bit-exact against the oracle's 8-bit append, the output within the
    tolerance of the oracle over the appended, dequantized cache."""
    torch = torch_cuda()
    R, maxL = len(lens), max(lens)
    b = build_batch(f"rand8f-{idx}", 1600 + idx, lens, [1] * R, num_blocks=sum(-(-L // 16) for L in lens) + 8,
                    num_layers=1, num_heads=heads, stride=-(-maxL // 16) + 1)
    codes, scales = ofp8.quantize_rows(b.pool)
    want_c, want_s = ofp8.append(codes, scales, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token,
                                 b.block_tables)
    ref = ofp8.decode(want_c, want_s, 0, b.q[0], b.block_tables, b.context_lens, SCALE)
    codes_d, scales_d = dev(codes, torch), dev(scales, torch)
    cache = pkv.PagedCache8(codes_d, scales_d)
    ws = torch.empty(max(pkv.decode_workspace_size_fp8(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
    say(f"random fused 8-bit decode {idx}: {heads} heads, {R} rows, longest {maxL}")
    pkv.decode_attention_append_fp8(cache, 0, out, dev(b.q[0], torch), dev(b.k_new[0], torch), dev(b.v_new[0], torch),
                                    dev(b.block_tables, torch), dev(b.context_lens, torch), maxL, SCALE, ws)
    torch.cuda.synchronize()
    assert np.array_equal(codes_d.cpu().numpy(), want_c)
    assert np.array_equal(scales_d.cpu().numpy().view(np.uint32), np.asarray(want_s).view(np.uint32))
    assert_close(host_f64(out), ref, f"random fused 8-bit shape {idx}")
