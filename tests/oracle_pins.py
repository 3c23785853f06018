"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin is a function that raises AssertionError when the oracle is wrong.
They look up oracle functions through the module at call time, so the mutant
tests can plant a mistake in the oracle and show that some pin catches it.

The flat element offset of the pool layout, written out here independently of
the oracle's multi-dimensional indexing, is

    ((((b * NL + l) * 2 + kv) * H + h) * 16 + s) * D + d

for block b, layer l, kv in {0: key, 1: value}, head h, slot s, dim d
(LLM inference batching, faangrind, data model: [layers, 2, heads, 16, 128]
per block).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.blocks as oblocks
import oracle.brute as brute
import oracle.fp8 as ofp8
import oracle.paged as paged
import oracle.pool as opool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def flat_offset(b, l, kv, h, s, d, NL, H, D):
    return ((((b * NL + l) * 2 + kv) * H + h) * 16 + s) * D + d


def _page_in_flat(num_blocks, NL, H, D, layer, table, K, V, fill=np.uint16(0x7E00)):
    """Write contiguous K/V ([H, L, D] uint16) into a flat pool with explicit offsets."""
    L = K.shape[1]
    flat = np.full(num_blocks * NL * 2 * H * 16 * D, fill, dtype=np.uint16)
    dd = np.arange(D)
    for h in range(H):
        for j in range(L):
            b = int(table[j // 16])
            s = j % 16
            flat[flat_offset(b, layer, 0, h, s, 0, NL, H, D) + dd] = K[h, j]
            flat[flat_offset(b, layer, 1, h, s, 0, NL, H, D) + dd] = V[h, j]
    return flat.reshape(num_blocks, NL, 2, H, 16, D)


def _rand_bits(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16).view(np.uint16)


def _f64(bits):
    return np.asarray(bits).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- pool arithmetic

def pin_block_arithmetic():
    g = golden()
    three = g["three_requests_rounding"]
    per = [opool.blocks_needed(n) for n in three["lengths"]]
    assert per == three["block_size_16"]["per_request"]
    assert sum(per) == three["block_size_16"]["blocks"]
    assert sum(per) * 16 == three["block_size_16"]["slots"]
    assert sum(per) * 16 - sum(three["lengths"]) == three["block_size_16"]["unused_slots"]
    assert sum(three["lengths"]) == three["logical_tokens"]
    per4 = [opool.blocks_needed(n, 4) for n in three["lengths"]]
    assert sum(per4) == three["block_size_4"]["table_entries"]
    assert sum(per4) * 4 == three["block_size_4"]["slots"]
    p600 = g["paged_600_tokens"]
    nb = opool.blocks_needed(p600["tokens"])
    assert nb == p600["blocks"] and nb * 16 == p600["slots"]
    assert nb * 16 - p600["tokens"] == p600["wasted_slots"]
    assert nb * 16 * p600["bytes_per_token"] == p600["bytes"]
    assert opool.blocks_needed(g["request_2300_tokens"]["tokens"]) == g["request_2300_tokens"]["blocks"]


def pin_pool_capacity():
    g = golden()["seven_b_pool"]
    # every block holds [layers, 2, heads, 16, head_dim] FP16
    block_shape = (g["layers"], 2, g["heads"], g["block_tokens"], g["head_dim"])
    assert int(np.prod(block_shape)) * g["bytes_per_element"] == g["bytes_per_block"]
    assert 2 * g["layers"] * g["heads"] * g["head_dim"] * g["bytes_per_element"] == g["bytes_per_token"]
    assert g["pool_bytes"] // g["bytes_per_block"] == g["num_blocks"]
    assert g["num_blocks"] * g["block_tokens"] == g["pool_tokens"]
    assert round(g["average_request_tokens"] * g["bytes_per_token"] / 1e9, 2) == g["average_request_gb"]
    assert round(g["max_request_tokens"] * g["bytes_per_token"] / 1e9, 2) == g["max_request_gb"]
    for tokens, fit in ((g["average_request_tokens"], g["average_requests_that_fit"]),
                        (g["max_request_tokens"], g["max_requests_that_fit"])):
        pool = opool.BlockPool(g["num_blocks"])
        count = 0
        while True:
            try:
                pool.alloc(opool.blocks_needed(tokens))
            except opool.OutOfBlocks:
                break
            count += 1
        assert count == fit, (tokens, count, fit)
    m = golden()["admission_margin"]
    assert round(m["fraction"] * g["num_blocks"]) == m["blocks"]


def pin_pool_semantics():
    # free list 0..N-1, pop() from the end, release appends in the order given
    p = opool.BlockPool(8)
    assert p.alloc(3) == [7, 6, 5]
    p.release([6, 7])
    assert p.free == [0, 1, 2, 3, 4, 6, 7]
    assert p.alloc(1) == [7]
    # all or nothing
    before = list(p.free)
    try:
        p.alloc(len(before) + 1)
        raise AssertionError("over-allocation accepted")
    except opool.OutOfBlocks:
        pass
    assert p.free == before
    # shared blocks return only at count zero; over-release is refused with no change
    p.share([5])
    assert p.ref[5] == 2
    p.release([5])
    assert p.ref[5] == 1 and 5 not in p.free
    try:
        p.release([5, 5])
        raise AssertionError("double free accepted")
    except opool.DoubleFree:
        pass
    assert p.ref[5] == 1
    p.release([5])
    assert p.free[-1] == 5 and p.ref[5] == 0
    # grow: P5-style all-or-nothing growth of a table
    t = []
    assert p.grow(t, 33) and len(t) == 3
    assert not p.grow(t, 16 * 100) and len(t) == 3


# ---------------------------------------------------------------- layout / append / gather

def pin_append_offsets(seed=11):
    rng = np.random.default_rng(seed)
    NB, NL, H, D = 9, 3, 2, 8
    pool = _rand_bits(rng, (NB, NL, 2, H, 16, D))
    table = np.array([[4, 1, 7], [0, 8, 2]], dtype=np.int32)
    positions = np.array([0, 15, 16, 33, 17, 47], dtype=np.int32)
    rows = np.array([0, 0, 0, 0, 1, 1], dtype=np.int32)
    k = _rand_bits(rng, (6, H, D))
    v = _rand_bits(rng, (6, H, D))
    layer = 2
    got = paged.append(pool, layer, k, v, positions, rows, table).reshape(-1)
    want = pool.reshape(-1).copy()
    for t in range(6):
        b = int(table[rows[t], positions[t] // 16])
        s = int(positions[t] % 16)
        for h in range(H):
            for d in range(D):
                want[flat_offset(b, layer, 0, h, s, d, NL, H, D)] = k[t, h, d]
                want[flat_offset(b, layer, 1, h, s, d, NL, H, D)] = v[t, h, d]
    assert np.array_equal(got, want)


def pin_gather_roundtrip(seed=12):
    rng = np.random.default_rng(seed)
    NB, NL, H, D = 12, 2, 3, 8
    for L in (1, 5, 16, 17, 40):
        table = rng.permutation(NB)[: -(-L // 16)].astype(np.int32)
        K = _rand_bits(rng, (H, L, D))
        V = _rand_bits(rng, (H, L, D))
        pool = _page_in_flat(NB, NL, H, D, 1, table, K, V)
        gk, gv = paged.gather_kv(pool[:, 1], table, L)
        assert gk.shape == (H, L, D)
        assert np.array_equal(gk, _f64(K)) and np.array_equal(gv, _f64(V))


# ---------------------------------------------------------------- attention

def pin_bruteforce(seed=13):
    rng = np.random.default_rng(seed)
    for H, D, lens, qn in ((1, 4, [1, 3, 17], [1, 2, 5]), (2, 8, [16, 33], [1, 8]), (32, 128, [20], [3])):
        NB = sum(-(-L // 16) for L in lens) + 2
        NL = 1
        ids = rng.permutation(NB)
        pos = 0
        tables = np.zeros((len(lens), 4), dtype=np.int32)
        conts = []
        pool = np.full((NB, NL, 2, H, 16, D), np.uint16(0x7E00), dtype=np.uint16)
        for r, L in enumerate(lens):
            nb = -(-L // 16)
            tables[r, :nb] = ids[pos:pos + nb]
            pos += nb
            K = _rand_bits(rng, (H, L, D))
            V = _rand_bits(rng, (H, L, D))
            sub = _page_in_flat(NB, NL, H, D, 0, tables[r], K, V, fill=np.uint16(0))
            used = np.zeros(NB, dtype=bool)
            used[tables[r, :nb]] = True
            pool[used] = sub[used]
            conts.append((K, V))
        qs = np.concatenate([[0], np.cumsum(qn)])
        q = _rand_bits(rng, (int(qs[-1]), H, D))
        scale = 1.0 / math.sqrt(D)
        out = paged.chunked_prefill(pool[:, 0], q, qs, tables, lens, scale)
        for r, L in enumerate(lens):
            K, V = (_f64(x) for x in conts[r])
            n = qn[r]
            for i in range(n):
                p = L - n + i
                for h in range(H):
                    want = brute.attend_one(list(_f64(q[qs[r] + i, h])), [list(K[h, j]) for j in range(p + 1)],
                                            [list(V[h, j]) for j in range(p + 1)], scale)
                    np.testing.assert_allclose(out[qs[r] + i, h], want, rtol=0, atol=1e-12)


def pin_closed_forms(seed=14):
    rng = np.random.default_rng(seed)
    H, D = 2, 8
    # hand-worked: q = e0, keys e0 and e1, values (1,2..) and (3,4..), scale 1 -> (e*v0 + v1) / (e + 1)
    q = np.zeros((1, 1, 2))
    q[0, 0, 0] = 1.0
    K = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    V = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    out = paged.attention(q, K, V, [1], 1.0)[0, 0]
    e = math.e
    np.testing.assert_allclose(out, [(e * 1 + 3) / (e + 1), (e * 2 + 4) / (e + 1)], rtol=1e-15)
    # the same query at position 0 sees only key 0 -> v0
    np.testing.assert_array_equal(paged.attention(q, K, V, [0], 1.0)[0, 0], V[0, 0])
    # a scale of 2 doubles the score gap
    out2 = paged.attention(q, K, V, [1], 2.0)[0, 0]
    np.testing.assert_allclose(out2, [(e ** 2 * 1 + 3) / (e ** 2 + 1), (e ** 2 * 2 + 4) / (e ** 2 + 1)], rtol=1e-15)
    # context of length 1 returns V exactly
    K1 = _f64(_rand_bits(rng, (H, 1, D)))
    V1 = _f64(_rand_bits(rng, (H, 1, D)))
    q1 = _f64(_rand_bits(rng, (1, H, D)))
    np.testing.assert_array_equal(paged.attention(q1, K1, V1, [0], 0.3)[0], V1[:, 0])
    # q = 0: uniform weights -> mean of the values
    L = 13
    Kr = _f64(_rand_bits(rng, (H, L, D)))
    Vr = _f64(_rand_bits(rng, (H, L, D)))
    np.testing.assert_allclose(paged.attention(np.zeros((1, H, D)), Kr, Vr, [L - 1], 0.3)[0], Vr.mean(axis=1),
                               rtol=0, atol=1e-14)
    # row-constant V returns the constant
    Vc = np.full((H, L, D), 0.625)
    np.testing.assert_allclose(paged.attention(q1, Kr, Vc, [L - 1], 0.3)[0], 0.625, rtol=0, atol=1e-15)
    # one key dominating by a gap g returns its value within (L-1) e^-g max|V|
    Kd = np.zeros((1, L, 2))
    Kd[0, 5, 0] = 30.0
    qd = np.array([[[1.0, 0.0]]])
    Vd = _f64(_rand_bits(rng, (1, L, 2)))
    got = paged.attention(qd, Kd, Vd, [L - 1], 1.0)[0, 0]
    assert np.max(np.abs(got - Vd[0, 5])) <= (L - 1) * math.exp(-30.0) * np.max(np.abs(Vd)) * 2


def pin_decode_reads_own_token(seed=15):
    g = golden()["decode_reads_own_token"]
    rng = np.random.default_rng(seed)
    H, D = 1, 8
    L = g["cache_after_step_1"]
    table = np.arange(-(-L // 16), dtype=np.int32)
    K = np.zeros((H, L, D), dtype=np.float16)
    V = np.zeros((H, L, D), dtype=np.float16)
    V[0, L - 1] = 1.0          # only the newest position carries value
    K[0, L - 1, 0] = 8.0       # and it wins the softmax by a wide margin
    pool = _page_in_flat(len(table), 1, H, D, 0, table, K.view(np.uint16), V.view(np.uint16), fill=np.uint16(0))
    q = np.zeros((1, H, D), dtype=np.float16)
    q[0, 0, 0] = 8.0
    out = paged.decode(pool[:, 0], q.view(np.uint16), table[None, :], [L], 1.0)
    gk, _ = paged.gather_kv(pool[:, 0], table, L)
    assert gk.shape[1] == g["positions_read_in_step_1"]
    assert out[0, 0, 0] > 0.99
    assert g["prompt_tokens"] + g["answer_tokens"] - 1 == g["final_cache"]


def pin_invariants(seed=16):
    rng = np.random.default_rng(seed)
    H, D, NB = 2, 16, 24
    lens = [37, 16, 5]
    nbs = [-(-L // 16) for L in lens]
    pool = _rand_bits(rng, (NB, 1, 2, H, 16, D))
    tables = np.zeros((3, 3), dtype=np.int32)
    ids = rng.permutation(NB)
    pos = 0
    for r, nb in enumerate(nbs):
        tables[r, :nb] = ids[pos:pos + nb]
        pos += nb
    q = _rand_bits(rng, (3, H, D))
    base = paged.decode(pool[:, 0], q, tables, lens, 0.25)
    # permuting physical ids (moving block contents with them) changes nothing, bit for bit
    perm = rng.permutation(NB)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    tables2 = perm[tables].astype(np.int32)
    np.testing.assert_array_equal(paged.decode(pool2[:, 0], q, tables2, lens, 0.25), base)
    # a prefix shared through the same ids equals private copies of it
    shared = tables.copy()
    shared[1, 0] = tables[0, 0]
    priv_pool = pool.copy()
    priv_pool[tables[1, 0]] = pool[tables[0, 0]]
    np.testing.assert_array_equal(paged.decode(pool[:, 0], q, shared, lens, 0.25),
                                  paged.decode(priv_pool[:, 0], q, tables, lens, 0.25))
    # adding one vector u to every key shifts every score equally
    K, V = paged.gather_kv(pool[:, 0], tables[0], lens[0])
    u = rng.standard_normal((H, 1, D))
    qf = _f64(q[0:1])
    a = paged.attention(qf, K, V, [lens[0] - 1], 0.25)
    b = paged.attention(qf, K + u, V, [lens[0] - 1], 0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # a chunk of one query is a decode; chunk query i equals a decode over its prefix
    qs = np.array([0, 4, 5, 6])
    qc = _rand_bits(rng, (6, H, D))
    pre = paged.chunked_prefill(pool[:, 0], qc, qs, tables, lens, 0.25)
    for i in range(4):
        p = lens[0] - 4 + i
        one = paged.decode(pool[:, 0], qc[i:i + 1], tables[0:1], [p + 1], 0.25)
        # equal up to the summation order of the library matmul
        np.testing.assert_allclose(pre[i], one[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(pre[4], paged.decode(pool[:, 0], qc[4:5], tables[1:2], [lens[1]], 0.25)[0],
                               rtol=0, atol=1e-14)


def pin_copy_on_write_divergence(seed=17):
    """Two branches share a 20-token prefix (one full block and one partial
    block, both layers).  Branch B copies the partial block before writing its
    own token 20 into the copy; branch A writes its token 20 into the shared
    original.  Each branch's decode, in both layers, must equal brute-force
    attention over its own contiguous context, which never passed through a
    block table or a copy."""
    rng = np.random.default_rng(seed)
    NB, NL, H, D = 10, 2, 2, 8
    a_blk, b_blk, c_blk = 6, 2, 9
    prefix = [_rand_bits(rng, (2, H, 20, D)) for _ in range(NL)]  # per layer: K, V of the shared prefix
    tokA = [_rand_bits(rng, (2, H, 1, D)) for _ in range(NL)]
    tokB = [_rand_bits(rng, (2, H, 1, D)) for _ in range(NL)]
    pool = None
    for l in range(NL):
        lay = _page_in_flat(NB, NL, H, D, l, [a_blk, b_blk], prefix[l][0], prefix[l][1])
        pool = lay if pool is None else pool
        pool[:, l] = lay[:, l]
    pool = oblocks.copy_blocks(pool, [b_blk], [c_blk])
    tables = np.array([[a_blk, b_blk], [a_blk, c_blk]], dtype=np.int32)
    for l in range(NL):
        kn = np.stack([tokA[l][0][:, 0], tokB[l][0][:, 0]])
        vn = np.stack([tokA[l][1][:, 0], tokB[l][1][:, 0]])
        pool = paged.append(pool, l, kn, vn, [20, 20], [0, 1], tables)
    q = _rand_bits(rng, (2, H, D))
    for l in range(NL):
        got = paged.decode(pool[:, l], q, tables, [21, 21], 0.25)
        for r, tok in enumerate((tokA, tokB)):
            K = np.concatenate([prefix[l][0], tok[l][0]], axis=1)
            V = np.concatenate([prefix[l][1], tok[l][1]], axis=1)
            for h in range(H):
                ref = brute.attend_one(_f64(q[r, h]).tolist(), _f64(K[h]).tolist(), _f64(V[h]).tolist(), 0.25)
                np.testing.assert_allclose(got[r, h], ref, rtol=0, atol=1e-12)


def pin_swap_roundtrip(seed=18):
    """A host image holds each swapped block as the block's flat element range
    (checked with the independent offset formula), and restoring it at other
    physical ids, with the table remapped, leaves every decode output equal
    bit for bit, in every layer."""
    rng = np.random.default_rng(seed)
    NB, NL, H, D = 12, 2, 2, 8
    pool = _rand_bits(rng, (NB, NL, 2, H, 16, D))
    ids = [3, 7, 8, 1]
    host = oblocks.swap_out(pool, ids)
    flat = pool.reshape(-1)
    host_flat = host.reshape(len(ids), -1)
    per_block = NL * 2 * H * 16 * D
    assert host_flat.shape[1] == per_block
    for i, b in enumerate(ids):
        for l, kv, h, s_, d in ((0, 0, 0, 0, 0), (1, 1, 1, 15, D - 1), (1, 0, 1, 7, 3), (0, 1, 0, 9, 5)):
            assert host_flat[i, flat_offset(0, l, kv, h, s_, d, NL, H, D)] == flat[flat_offset(b, l, kv, h, s_, d, NL, H, D)]
    new_ids = [5, 0, 11, 2]
    poisoned = pool.copy()
    poisoned[new_ids] = np.uint16(0x7E00)
    restored = oblocks.swap_in(poisoned, host, new_ids)
    remap = {o: n for o, n in zip(ids, new_ids)}
    tables = np.array([[3, 7], [8, 1]], dtype=np.int32)
    tables2 = np.vectorize(remap.get)(tables).astype(np.int32)
    q = _rand_bits(rng, (2, H, D))
    for l in range(NL):
        np.testing.assert_array_equal(paged.decode(restored[:, l], q, tables2, [29, 20], 0.25),
                                      paged.decode(pool[:, l], q, tables, [29, 20], 0.25))


def pin_grouped_query(seed=19):
    """Grouped-query attention: with KV heads shared by groups of 4 query
    heads, decode and prefill equal plain multi-head attention over a pool
    whose every query head holds its own copy of KV head h // 4 (written with
    the independent flat offsets), and brute force with that mapping spelled
    out."""
    rng = np.random.default_rng(seed)
    Hkv, G, D, NB = 2, 4, 8, 12
    Hq = Hkv * G
    lens = [20, 5]
    tables = np.array([[7, 3], [10, 0]], dtype=np.int32)
    K = [_rand_bits(rng, (Hkv, L, D)) for L in lens]
    V = [_rand_bits(rng, (Hkv, L, D)) for L in lens]
    gqa = None
    mha = None
    for r, L in enumerate(lens):
        a = _page_in_flat(NB, 1, Hkv, D, 0, tables[r], K[r], V[r])
        dup = np.array([h // G for h in range(Hq)])
        b = _page_in_flat(NB, 1, Hq, D, 0, tables[r], K[r][dup], V[r][dup])
        gqa = a if gqa is None else np.where(np.isin(np.arange(NB), tables[r][:-(-L // 16)])[:, None, None, None, None, None], a, gqa)
        mha = b if mha is None else np.where(np.isin(np.arange(NB), tables[r][:-(-L // 16)])[:, None, None, None, None, None], b, mha)
    q = _rand_bits(rng, (2, Hq, D))
    got = paged.decode(gqa[:, 0], q, tables, lens, 0.3, group=G)
    np.testing.assert_array_equal(got, paged.decode(mha[:, 0], q, tables, lens, 0.3))
    for r, L in enumerate(lens):
        for h in range(Hq):
            ref = brute.attend_one(_f64(q[r, h]).tolist(), _f64(K[r][h // G]).tolist(), _f64(V[r][h // G]).tolist(), 0.3)
            np.testing.assert_allclose(got[r, h], ref, rtol=0, atol=1e-12)
    qs = np.array([0, 3, 4])
    qc = _rand_bits(rng, (4, Hq, D))
    np.testing.assert_array_equal(paged.chunked_prefill(gqa[:, 0], qc, qs, tables, lens, 0.3, group=G),
                                  paged.chunked_prefill(mha[:, 0], qc, qs, tables, lens, 0.3))


def pin_fp8_format(seed=20):
    """E4M3 codes as the OCP 8-bit floating point format defines them (one sign,
    four exponent bits with bias 7, three mantissa bits, no infinity, 0x7F NaN):
    spot values, ties to the even mantissa, saturation at 448, and the encoder
    against a brute-force nearest-code search."""
    t = ofp8.decode_table()
    for code, val in ((0x00, 0.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x3A, 1.25), (0x40, 2.0),
                      (0x7E, 448.0), (0xC0, -2.0), (0x46, 3.5)):
        assert t[code] == val, (hex(code), t[code], val)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    enc = lambda x: int(ofp8.encode(np.float32(x)))
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A      # halfway: to the even mantissa
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02  # subnormal ties
    assert enc(1000.0) == 0x7E and enc(-1e6) == 0xFE and enc(464.0) == 0x7E  # saturation
    finite = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert np.array_equal(ofp8.encode(t[finite].astype(np.float32)), finite.astype(np.uint8))
    # an independent implementation: torch's CPU conversion to float8_e4m3fn
    # rounds to nearest even and agrees with the definition below 464 (above
    # that it gives NaN where the reading saturates)
    import torch
    rng = np.random.default_rng(seed)
    xs = np.concatenate([rng.uniform(-463, 463, 20000), rng.uniform(-0.05, 0.05, 20000),
                         rng.standard_normal(20000) * 8, (t[finite][:-1] + t[finite][1:]) / 2,
                         np.nextafter((t[finite][:-1] + t[finite][1:]) / 2, 0)]).astype(np.float32)
    xs = xs[np.abs(xs) < 464]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ofp8.encode(xs), ref)
    # brute force: the nearest finite code, ties to the even code
    xs = np.concatenate([rng.uniform(-460, 460, 3000), rng.uniform(-0.03, 0.03, 3000),
                         (t[finite][:-1] + t[finite][1:]) / 2]).astype(np.float32)
    vals = t[finite]
    for x in xs[:: 7]:
        if abs(float(x)) >= 448.0:
            continue
        d = np.abs(vals - float(x))
        best = np.flatnonzero(d == d.min())
        cands = finite[best]
        if len(cands) > 1:  # a tie between two neighbours: the one with the even mantissa
            cands = [c for c in cands if (c & 1) == 0] or cands
        want = {int(c) for c in cands}
        # +0 / -0 both encode a zero
        got = enc(x)
        assert got in want or (t[got] == 0 and 0.0 in vals[best]), (float(x), hex(got), [hex(c) for c in want])


def pin_fp8_quantized_cache(seed=21):
    """Per-(token, head) quantization: every element within the format's
    half-step of its value, each row's largest magnitude restored to fp32
    rounding, zero rows kept, codes placed by the FP16 append's rule, and
    decode over the cache equal to brute force over the dequantized values."""
    rng = np.random.default_rng(seed)
    H, D = 2, 128
    x = _rand_bits(rng, (5, H, D))
    x[2, 1] = 0  # a zero row
    codes, sc = ofp8.quantize_rows(x)
    xf = _f64(x)
    deq = ofp8.dequantize(codes, sc)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * sc[..., None] + 1e-12)
    assert np.all(np.abs(deq - xf) <= bound * (1 + 1e-6))
    amax = np.abs(xf).max(axis=-1)
    rows = np.argmax(np.abs(xf), axis=-1)
    got_max = np.take_along_axis(np.abs(deq), rows[..., None], axis=-1)[..., 0]
    np.testing.assert_allclose(got_max, amax, rtol=2e-7, atol=0)
    assert sc[2, 1] == 0 and not codes[2, 1].any()
    # append places codes exactly where the FP16 append places values
    NB, NL = 6, 2
    cp = np.zeros((NB, NL, 2, H, 16, D), dtype=np.uint8)
    sp = np.zeros((NB, NL, 2, H, 16), dtype=np.float32)
    tables = np.array([[4, 1], [0, 5]], dtype=np.int32)
    k, v = _rand_bits(rng, (3, H, D)), _rand_bits(rng, (3, H, D))
    cp, sp = ofp8.append(cp, sp, 1, k, v, [17, 0, 31], [0, 1, 1], tables)
    kc, ks = ofp8.quantize_rows(k)
    for t, (r, pos) in enumerate(((0, 17), (1, 0), (1, 31))):
        b, slot = int(tables[r, pos // 16]), pos % 16
        assert np.array_equal(cp[b, 1, 0, :, slot], kc[t]) and np.array_equal(sp[b, 1, 0, :, slot], ks[t])
    # decode over the cache: brute force over dequantized contiguous values
    L = 20
    ck = rng.integers(0, 0x7E, (H, L, D)).astype(np.uint8)
    cv = rng.integers(0, 0x7E, (H, L, D)).astype(np.uint8) | (rng.integers(0, 2, (H, L, D)).astype(np.uint8) << 7)
    sk = rng.uniform(0.001, 0.01, (H, L)).astype(np.float32)
    sv = rng.uniform(0.001, 0.01, (H, L)).astype(np.float32)
    pool_c = np.zeros((4, 1, 2, H, 16, D), dtype=np.uint8)
    pool_s = np.zeros((4, 1, 2, H, 16), dtype=np.float32)
    tab = np.array([[3, 0]], dtype=np.int32)
    for j in range(L):
        b, slot = int(tab[0, j // 16]), j % 16
        pool_c[b, 0, 0, :, slot], pool_c[b, 0, 1, :, slot] = ck[:, j], cv[:, j]
        pool_s[b, 0, 0, :, slot], pool_s[b, 0, 1, :, slot] = sk[:, j], sv[:, j]
    q = _rand_bits(rng, (1, H, D))
    got = ofp8.decode(pool_c, pool_s, 0, q, tab, [L], 0.25)
    table = ofp8.decode_table()
    for h in range(H):
        Kd = [[table[ck[h, j, d]] * float(sk[h, j]) for d in range(D)] for j in range(L)]
        Vd = [[table[cv[h, j, d]] * float(sv[h, j]) for d in range(D)] for j in range(L)]
        ref = brute.attend_one(_f64(q[0, h]).tolist(), Kd, Vd, 0.25)
        np.testing.assert_allclose(got[0, h], ref, rtol=0, atol=1e-12)


ALL_PINS = [pin_block_arithmetic, pin_pool_capacity, pin_pool_semantics, pin_append_offsets,
            pin_gather_roundtrip, pin_bruteforce, pin_closed_forms, pin_decode_reads_own_token, pin_invariants,
            pin_copy_on_write_divergence, pin_swap_roundtrip, pin_grouped_query, pin_fp8_format,
            pin_fp8_quantized_cache]
