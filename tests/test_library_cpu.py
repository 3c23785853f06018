"""libpkv.so on the CPU: it loads, exports every symbol pkv.h declares, the
host pool matches the oracle's pool model, and argument validation rejects
bad calls before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle.pool as opool
import paged_kv_cache_pkv_amd as pkv
from paged_kv_cache_pkv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with pkv.h"


def test_version_and_constants():
    assert "gfx950" in pkv.version()
    assert pkv.split_tokens() % 16 == 0
    for n, want in ((0, 0), (1, 1), (16, 1), (17, 2), (600, 38), (2300, 144), (8192, 512)):
        assert pkv.blocks_needed(n) == want == opool.blocks_needed(n)


def test_pool_matches_model_fuzz():
    rng = np.random.default_rng(5)
    for trial in range(6):
        N = int(rng.integers(1, 300))
        perm = rng.permutation(N) if trial % 2 else None
        nfree = N if perm is None else int(rng.integers(0, N + 1))
        fl = None if perm is None else perm[:nfree]
        lib_pool = pkv.BlockPool(N, fl)
        model = opool.BlockPool(N, fl)
        held = [b for b in range(N) if model.ref[b] > 0]
        for step in range(400):
            op = rng.integers(0, 4)
            if op == 0:
                n = int(rng.integers(0, 12))
                try:
                    want = model.alloc(n)
                except opool.OutOfBlocks:
                    with pytest.raises(pkv.PkvError) as e:
                        lib_pool.alloc(n)
                    assert e.value.name == "OUT_OF_BLOCKS"
                else:
                    got = lib_pool.alloc(n)
                    assert list(got) == want
                    held.extend(want)
            elif op == 1 and held:
                ids = list(rng.choice(held, size=min(len(held), int(rng.integers(1, 5))), replace=True))
                try:
                    model.release(ids)
                except opool.DoubleFree:
                    with pytest.raises(pkv.PkvError) as e:
                        lib_pool.free(ids)
                    assert e.value.name == "DOUBLE_FREE"
                else:
                    lib_pool.free(ids)
                held = [b for b in range(N) if model.ref[b] > 0]
            elif op == 2 and held:
                ids = list(rng.choice(held, size=min(len(held), 3), replace=False))
                model.share(ids)
                lib_pool.ref(ids)
            elif op == 3:
                b = int(rng.integers(0, N))
                if model.ref[b] == 0:
                    with pytest.raises(pkv.PkvError) as e:
                        lib_pool.free([b])
                    assert e.value.name == "DOUBLE_FREE"
            assert lib_pool.num_free == model.num_free()
            assert list(lib_pool.free_list()) == model.free
        assert [lib_pool.ref_count(b) for b in range(N)] == model.ref
        lib_pool.close()


def test_pool_pages_arithmetic_and_drain():
    # the faangrind 7B pool: 7,152 blocks; 73 average (1,550-token) requests fit, 13 at 8,192
    for tokens, fit in ((1550, 73), (8192, 13)):
        p = pkv.BlockPool(7152)
        tables = []
        while True:
            try:
                tables.append(p.alloc(pkv.blocks_needed(tokens)))
            except pkv.PkvError as e:
                assert e.name == "OUT_OF_BLOCKS"
                break
        assert len(tables) == fit
        for t in tables:
            p.free(t)
        assert p.num_free == 7152  # drain returns every block


def test_pool_grow_and_shared_prefix():
    p = pkv.BlockPool(64, np.random.default_rng(0).permutation(64))
    t = np.zeros(16, dtype=np.int32)
    n = p.grow(t, 0, 17)
    assert n == 2 and p.num_free == 62
    n = p.grow(t, n, 32)
    assert n == 2
    n = p.grow(t, n, 33)
    assert n == 3
    with pytest.raises(pkv.PkvError) as e:
        p.grow(t, n, 16 * 100)
    assert e.value.name == "INVALID_ARG"  # capacity 16 blocks
    big = np.zeros(100, dtype=np.int32)
    with pytest.raises(pkv.PkvError) as e:
        p.grow(big, 0, 16 * 62)
    assert e.value.name == "OUT_OF_BLOCKS" and p.num_free == 61
    # a second row shares the first two blocks
    p.ref(t[:2])
    assert p.ref_count(int(t[0])) == 2
    p.free(t[:3])
    assert p.ref_count(int(t[0])) == 1 and p.num_free == 62
    p.free(t[:2])
    assert p.num_free == 64


def test_pool_bad_arguments():
    with pytest.raises(pkv.PkvError):
        pkv.BlockPool(0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.BlockPool(4, [0, 0])
    assert e.value.name == "BAD_BLOCK"
    p = pkv.BlockPool(4)
    with pytest.raises(pkv.PkvError) as e:
        p.free([7])
    assert e.value.name == "BAD_BLOCK"
    with pytest.raises(pkv.PkvError) as e:
        p.ref([1])
    assert e.value.name == "DOUBLE_FREE"
    assert p.ref_count(9) == -1


def _desc(**kw):
    d = dict(base=ctypes.c_void_p(0x100000), num_blocks=64, num_layers=1, num_heads=32, block_size=16, head_dim=128)
    d.update(kw)
    return _lib.PkvCacheDesc(d["base"], d["num_blocks"], d["num_layers"], d["num_heads"], d["block_size"],
                             d["head_dim"])


FAKE = ctypes.c_void_p(0x200000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), -2), (dict(block_size=32), -2), (dict(num_heads=0), -2),
    (dict(base=ctypes.c_void_p(0)), -1), (dict(num_layers=0), -1),
])
def test_validation_cache(kw, code):
    L = pkv.lib()
    d = _desc(**kw)
    rc = L.pkv_decode_attention(ctypes.byref(d), 0, FAKE, FAKE, FAKE, 16, FAKE, 4, 256, 0.088, FAKE, 1 << 20, None)
    assert rc == code
    assert L.pkv_last_error()
    rc = L.pkv_append(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 16, None)
    assert rc == code


def test_validation_decode_args():
    L = pkv.lib()
    d = _desc()
    args = lambda **k: dict(dict(layer=0, out=FAKE, q=FAKE, bt=FAKE, stride=16, cl=FAKE, R=4, maxL=256, scale=0.088,
                                 ws=FAKE, wsb=1 << 20), **k)
    def call(a):
        return L.pkv_decode_attention(ctypes.byref(d), a["layer"], a["out"], a["q"], a["bt"], a["stride"], a["cl"],
                                      a["R"], a["maxL"], a["scale"], a["ws"], a["wsb"], None)
    assert call(args(layer=1)) == -1
    assert call(args(R=0)) == -1
    assert call(args(maxL=0)) == -1
    assert call(args(maxL=16 * 16 + 1)) == -1
    assert call(args(out=None)) == -1
    assert call(args(scale=float("nan"))) == -1
    assert call(args(scale=-1.0)) == -1
    assert call(args(q=ctypes.c_void_p(0x200002))) == -1  # misaligned
    need = L.pkv_decode_workspace_size(ctypes.byref(d), 4, 4096)
    assert need > 0
    assert call(args(stride=256, maxL=4096, ws=None)) == -6
    assert call(args(stride=256, maxL=4096, wsb=need - 1)) == -6
    assert call(args(stride=256, maxL=4096, ws=ctypes.c_void_p(0x200010), wsb=need)) == -6  # 256-B alignment


def test_validation_append_args():
    L = pkv.lib()
    d = _desc()
    assert L.pkv_append(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 4, 16, None) == 0  # empty = no-op
    assert L.pkv_append(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 4, 16, None) == -1
    assert L.pkv_append(ctypes.byref(d), 2, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 16, None) == -1
    assert L.pkv_append(ctypes.byref(d), 0, None, FAKE, FAKE, FAKE, 4, FAKE, 4, 16, None) == -1
    assert L.pkv_append(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0, 16, None) == -1


def test_validation_prefix_decode():
    L = pkv.lib()
    d = _desc()

    def call(P, shares=FAKE, stride=16, maxL=256, ws=FAKE, wsb=1 << 20, **k):
        return L.pkv_decode_attention_prefix(ctypes.byref(d), k.get("layer", 0), FAKE, FAKE, FAKE, stride, FAKE, 4,
                                             maxL, 0.088, shares, P, ws, wsb, None)
    assert call(-1) == -1
    assert call(17) == -1            # more prefix blocks than table entries
    assert call(3, shares=None) == -1
    assert call(2, layer=1) == -1
    # the workspace covers the prefix's ranges and a whole context's ranges
    plain = L.pkv_decode_workspace_size(ctypes.byref(d), 4, 4096)
    assert L.pkv_decode_workspace_size_prefix(ctypes.byref(d), 4, 4096, 0) == plain
    need = L.pkv_decode_workspace_size_prefix(ctypes.byref(d), 4, 4096, 125)
    per_range = 4 * 32 * (128 * 4 + 8)
    assert need >= plain + 8 * per_range - 512
    assert L.pkv_decode_workspace_size_prefix(ctypes.byref(d), 4, 4096, -1) == 0
    assert call(125, stride=256, maxL=4096, wsb=need - 1) == -6
    assert call(125, stride=256, maxL=4096, ws=None) == -6


def test_validation_check_tables():
    L = pkv.lib()
    d = _desc()

    def call(R=4, stride=16, maxL=256, bt=FAKE, cl=FAKE, qs=None, total_q=0, rep=FAKE, desc=d):
        return L.pkv_check_tables(ctypes.byref(desc), bt, stride, cl, R, maxL, qs, total_q, rep, None)
    assert call(R=0) == -1
    assert call(stride=0) == -1
    assert call(maxL=0) == -1
    assert call(maxL=16 * 16 + 1) == -1
    assert call(bt=None) == -1
    assert call(cl=None) == -1
    assert call(rep=None) == -1
    assert call(qs=FAKE, total_q=0) == -1  # query checks need the step's query count
    assert call(desc=_desc(head_dim=64)) == -2
    assert L.pkv_last_error()


def test_validation_block_copies():
    L = pkv.lib()
    d = _desc(num_layers=3, num_heads=5)
    assert L.pkv_block_bytes(ctypes.byref(d)) == 3 * 2 * 5 * 16 * 128 * 2
    bad = _desc(head_dim=64)
    assert L.pkv_block_bytes(ctypes.byref(bad)) == 0
    # copy-on-write pairs live on the device: only the scalars are checked here
    assert L.pkv_copy_blocks(ctypes.byref(d), FAKE, FAKE, 0, None) == 0  # empty = no-op
    assert L.pkv_copy_blocks(ctypes.byref(d), FAKE, FAKE, -1, None) == -1
    assert L.pkv_copy_blocks(ctypes.byref(d), None, FAKE, 2, None) == -1
    assert L.pkv_copy_blocks(ctypes.byref(bad), FAKE, FAKE, 2, None) == -2
    # swap ids live on the host and are all checked before anything is queued
    ids = np.array([3, 64, 1], dtype=np.int32)
    p = ids.ctypes.data_as(_lib.c_i32_p)
    assert L.pkv_swap_out(ctypes.byref(d), p, 3, FAKE, None) == -5
    assert b"64" in L.pkv_last_error()
    assert L.pkv_swap_in(ctypes.byref(d), FAKE, p, 3, None) == -5
    neg = np.array([-1], dtype=np.int32)
    assert L.pkv_swap_in(ctypes.byref(d), FAKE, neg.ctypes.data_as(_lib.c_i32_p), 1, None) == -5
    assert L.pkv_swap_out(ctypes.byref(d), p, 0, FAKE, None) == 0
    assert L.pkv_swap_out(ctypes.byref(d), p, -2, FAKE, None) == -1
    assert L.pkv_swap_out(ctypes.byref(d), p, 1, None, None) == -1
    assert L.pkv_swap_in(ctypes.byref(d), None, p, 1, None) == -1


def test_validation_appending_decodes():
    """The fused append + decode calls check their extra arguments before any
    launch, and otherwise validate exactly as the plain decode calls do."""
    L = pkv.lib()
    d = _desc(num_heads=8)

    def call(k=FAKE, v=FAKE, layer=0, R=4, maxL=256, Hq=None):
        if Hq is None:
            return L.pkv_decode_attention_append(ctypes.byref(d), layer, FAKE, FAKE, k, v, FAKE, 16, FAKE, R, maxL,
                                                 0.088, FAKE, 1 << 20, None)
        return L.pkv_decode_attention_append_gqa(ctypes.byref(d), Hq, layer, FAKE, FAKE, k, v, FAKE, 16, FAKE, R,
                                                 maxL, 0.088, FAKE, 1 << 20, None)
    assert call(k=None) == -1
    assert call(v=None) == -1
    assert call(k=ctypes.c_void_p(0x200008)) == -1  # misaligned new keys
    assert call(layer=1) == -1
    assert call(R=0) == -1
    assert call(maxL=16 * 16 + 1) == -1
    assert call(Hq=24) == -2    # 3 query heads per KV head is not a supported group
    assert call(Hq=8 * 16) == -2
    assert call(Hq=32, k=None) == -1
    assert L.pkv_decode_attention_append(None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 256, 0.088, FAKE, 1 << 20,
                                         None) == -1
    d8 = _lib.PkvCache8Desc(ctypes.c_void_p(0x100000), ctypes.c_void_p(0x300000), 64, 1, 32, 16, 128)
    assert L.pkv_decode_attention_append_fp8(ctypes.byref(d8), 0, FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, 4, 256,
                                             0.088, FAKE, 1 << 20, None) == -1
    assert L.pkv_decode_attention_append_fp8(ctypes.byref(d8), 0, FAKE, FAKE, ctypes.c_void_p(0x200004), FAKE, FAKE,
                                             16, FAKE, 4, 256, 0.088, FAKE, 1 << 20, None) == -1
    assert L.pkv_decode_attention_append_fp8(ctypes.byref(d8), 1, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 256,
                                             0.088, FAKE, 1 << 20, None) == -1


def test_binding_refuses_short_tensors():
    """The binding checks each tensor against the counts the call will index it
    by (rows x heads x 128 for queries and outputs, rows for lengths), before
    any library call: a short tensor would be read or written past its end."""
    torch = pytest.importorskip("torch")

    class Cache:  # only the head count is consulted before the refusal
        num_heads = 8
        desc = None

    R, H = 4, 8
    tables = torch.zeros((R, 16), dtype=torch.int32)
    lens = torch.ones(R, dtype=torch.int32)
    full = torch.zeros((R, H, 128), dtype=torch.float16)
    short = torch.zeros((R - 1, H, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="out has"):
        pkv.decode_attention_gqa(Cache(), H, 0, short, full, tables, lens, 64, 0.088)
    with pytest.raises(ValueError, match="q has"):
        pkv.decode_attention_gqa(Cache(), H, 0, full, short, tables, lens, 64, 0.088)
    with pytest.raises(ValueError, match="context_lens has"):
        pkv.decode_attention_gqa(Cache(), H, 0, full, full, tables, lens[:2], 64, 0.088)
    with pytest.raises(ValueError, match="out has"):  # 4 query heads per KV head need 4x the output rows
        pkv.decode_attention_gqa(Cache(), 4 * H, 0, full, full, tables, lens, 64, 0.088)
    with pytest.raises(ValueError, match="k_new has"):
        pkv.decode_attention_append(Cache(), 0, full, full, short, full, tables, lens, 64, 0.088)
    with pytest.raises(ValueError, match="shares_prefix has"):
        pkv.decode_attention_prefix(Cache(), 0, full, full, tables, lens, 64, 0.088, lens[:1], 2)
    pos = torch.zeros(R, dtype=torch.int32)
    with pytest.raises(ValueError, match="v_new has"):
        pkv.append(Cache(), 0, full, short, pos, pos, tables)
    with pytest.raises(ValueError, match="request_of_token has"):
        pkv.append(Cache(), 0, full, full, pos, pos[:1], tables)
    qs = torch.tensor([0, 1, 2, 3, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="out has"):
        pkv.chunked_prefill_attention(Cache(), 0, short, full, qs, tables, lens, 1, 64, 0.088)
    with pytest.raises(ValueError, match="query_start has"):
        pkv.chunked_prefill_attention(Cache(), 0, full, full, qs[:R], tables, lens, 1, 64, 0.088)
    with pytest.raises(ValueError, match="out has"):
        pkv.decode_attention_fp8(Cache(), 0, short, full, tables, lens, 64, 0.088)


def test_validation_chunked_prefill_args():
    """pkv_chunked_prefill_attention checks every scalar, pointer, alignment
    and workspace before it launches anything; its workspace size is the one
    of the grouped call with one query head per KV head."""
    L = pkv.lib()
    d = _desc()

    def call(layer=0, out=FAKE, q=FAKE, qs=FAKE, bt=FAKE, stride=16, cl=FAKE, R=4, T=40, maxq=32, maxL=256,
             scale=0.088, ws=FAKE, wsb=1 << 24, desc=None):
        return L.pkv_chunked_prefill_attention(ctypes.byref(desc or d), layer, out, q, qs, bt, stride, cl, R, T, maxq,
                                               maxL, scale, ws, wsb, None)
    need = L.pkv_prefill_workspace_size(ctypes.byref(d), 4, 40, 32, 256)
    assert need > 0
    assert need == L.pkv_prefill_workspace_size_gqa(ctypes.byref(d), 32, 4, 40, 32, 256)
    assert L.pkv_prefill_workspace_size(ctypes.byref(d), 4, 0, 32, 256) == 0
    assert L.pkv_prefill_workspace_size(None, 4, 40, 32, 256) == 0
    assert L.pkv_chunked_prefill_attention(None, 0, FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 40, 32, 256, 0.088, FAKE,
                                           1 << 24, None) == -1
    assert call(desc=_desc(head_dim=64)) == -2
    assert call(desc=_desc(block_size=8)) == -2
    assert call(layer=1) == -1 and call(layer=-1) == -1
    assert call(R=0) == -1
    assert call(T=0) == -1
    for k in ("out", "q", "qs", "bt", "cl"):
        assert call(**{k: None}) == -1, k
    assert call(stride=0) == -1
    assert call(maxL=0) == -1
    assert call(maxL=16 * 16 + 1) == -1                 # beyond the table
    assert call(maxq=0) == -1
    assert call(maxq=257) == -1                         # more queries than context
    assert call(T=20, maxq=32) == -1                    # more queries per row than in the call
    assert call(scale=float("nan")) == -1 and call(scale=0.0) == -1 and call(scale=float("inf")) == -1
    assert call(q=ctypes.c_void_p(0x200008)) == -1      # misaligned
    assert call(out=ctypes.c_void_p(0x200004)) == -1
    assert call(desc=_desc(base=ctypes.c_void_p(0x100002))) == -1
    assert call(ws=None) == -6
    assert call(wsb=need - 1) == -6
    assert call(ws=ctypes.c_void_p(0x200010), wsb=need) == -6  # 256-byte alignment
    assert b"workspace" in L.pkv_last_error()


def test_pool_grow_rows_matches_model():
    """pkv_grow_rows grows each row as the oracle pool model's grow does, rows
    in order, each all or nothing, stopping at the first row the free list
    cannot cover; bad arguments of any row change nothing."""
    rng = np.random.default_rng(23)
    N, R, stride = 120, 6, 12
    perm = rng.permutation(N).astype(np.int32)
    lib_pool = pkv.BlockPool(N, perm)
    model = opool.BlockPool(N, perm)
    tables = np.zeros((R, stride), dtype=np.int32)
    lens = np.zeros(R, dtype=np.int32)
    mtables = [[] for _ in range(R)]
    tokens = np.zeros(R, dtype=np.int64)
    for step in range(40):
        tokens += rng.integers(0, 40, R)
        tokens = np.minimum(tokens, 16 * stride)
        got = lib_pool.grow_rows(tables, lens, tokens)
        want = R
        for r in range(R):
            if not model.grow(mtables[r], int(tokens[r])):
                want = r
                break
        assert got == want
        for r in range(R):
            assert list(tables[r, :lens[r]]) == mtables[r]
        assert list(lib_pool.free_list()) == model.free
        if got < R:  # preempt the row that came up short: release it and start it over
            lib_pool.free(tables[got, :lens[got]])
            model.release(mtables[got])
            lens[got], mtables[got], tokens[got] = 0, [], 0
    before = (tables.copy(), lens.copy(), lib_pool.num_free)
    with pytest.raises(pkv.PkvError) as e:
        lib_pool.grow_rows(tables, lens, np.full(R, 16 * stride + 1))
    assert e.value.name == "INVALID_ARG"
    assert np.array_equal(tables, before[0]) and np.array_equal(lens, before[1]) and lib_pool.num_free == before[2]


def test_probe_library_exports_its_header():
    """The bandwidth and matrix-core probes (a measurement aid) export every call pkv_probe.h declares
    and reject bad arguments before any launch."""
    from paged_kv_cache_pkv_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pkv_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pkv_probe_[a-z0-9_]+)\s*\(", text)))
    assert names == sorted(probe.SIGNATURES)
    L = probe.lib()
    assert L.pkv_probe_stream_read(None, 4096, FAKE, 1, None) == -1
    assert L.pkv_probe_stream_read(FAKE, 4100, FAKE, 1, None) == -1     # not a multiple of 16
    assert L.pkv_probe_stream_read(FAKE, 1 << 31, FAKE, 1, None) == -1  # too large
    assert L.pkv_probe_slab_read(FAKE, 1 << 20, FAKE, 4, 4000, FAKE, 1, None) == -1  # slab not a multiple of 4096
    assert L.pkv_probe_slab_read(FAKE, 1 << 20, FAKE, -1, 4096, FAKE, 1, None) == -1
    assert L.pkv_probe_slab_read(FAKE, 1 << 20, FAKE, 0, 4096, FAKE, 1, None) == 0   # nothing to read
    flops = ctypes.c_double(0.0)
    assert L.pkv_probe_mfma_f16(0, FAKE, ctypes.byref(flops), None) == -1        # no rounds
    assert L.pkv_probe_mfma_f16((1 << 24) + 1, FAKE, ctypes.byref(flops), None) == -1
    assert L.pkv_probe_mfma_f16(10, None, ctypes.byref(flops), None) == -1
    assert L.pkv_probe_mfma_f16(10, FAKE, None, None) == -1
