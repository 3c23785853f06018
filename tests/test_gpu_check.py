"""pkv_check_tables on the GPU: the device report against the same counts taken
on the host, for clean steps, planted bad entries, long rows and a captured
graph replayed over changing inputs."""
import numpy as np
import pytest

import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, say, torch_cuda
from workloads import c2_average_mix

pytestmark = pytest.mark.gpu


def expected(tables, lens, max_len, num_blocks, query_start=None, total_q=0):
    """[bad lengths, bad table entries, bad query ranges, first bad row or -1],
    counted row by row as the header defines them."""
    bad_len = bad_id = bad_q = 0
    first = -1
    for r, L in enumerate(int(x) for x in lens):
        lb = L < 1 or L > max_len
        nb = -(-min(max(L, 0), max_len) // 16)
        ib = sum(1 for j in range(nb) if not 0 <= int(tables[r, j]) < num_blocks)
        qb = False
        if query_start is not None:
            q0, q1 = int(query_start[r]), int(query_start[r + 1])
            qb = q0 < 0 or q1 > total_q or q1 - q0 < 1 or q1 - q0 > L
        bad_len += lb
        bad_id += ib
        bad_q += qb
        if (lb or ib or qb) and first < 0:
            first = r
    return [bad_len, bad_id, bad_q, first]


def _cache(torch, num_blocks):
    # the check reads no pool bytes; a one-head, one-layer pool gives the descriptor
    pool = torch.empty((num_blocks, 1, 2, 1, 16, 128), dtype=torch.int16, device="cuda")
    return pool, pkv.PagedCache(pool)


def _run(torch, cache, tables, lens, max_len, query_start=None, total_q=0):
    report = torch.full((4,), 12345, dtype=torch.int32, device="cuda")
    pkv.check_tables(cache, dev(tables, torch), dev(lens, torch), max_len, report,
                     None if query_start is None else dev(query_start, torch), total_q)
    torch.cuda.synchronize()
    return [int(x) for x in report.cpu().numpy()]


def test_clean_average_mix_step():
    torch = torch_cuda()
    b = c2_average_mix(seed=1, with_pool=False)
    pool, cache = _cache(torch, 7152)
    max_len = b.bt_stride * 16
    say(f"check: average mix, {b.rows} rows, stride {b.bt_stride}")
    got = _run(torch, cache, b.block_tables, b.context_lens.astype(np.int32), max_len)
    assert got == [0, 0, 0, -1]


@pytest.mark.parametrize("seed,rows,stride", [(5, 37, 40), (6, 3, 600), (7, 70, 130)])
def test_planted_violations(seed, rows, stride):
    torch = torch_cuda()
    rng = np.random.default_rng(seed)
    nb_pool = 500
    max_len = stride * 16 - int(rng.integers(0, 16))
    lens = rng.integers(1, max_len + 1, size=rows).astype(np.int32)
    tables = rng.integers(0, nb_pool, size=(rows, stride)).astype(np.int32)
    # entries past each row's blocks are garbage the kernels never read
    for r in range(rows):
        tables[r, -(-int(lens[r]) // 16):] = rng.integers(-10**6, 10**6, size=stride - (-(-int(lens[r]) // 16)))
    # planted: bad lengths, bad ids inside used blocks (first, last, middle)
    picks = rng.choice(rows, size=min(rows, 6), replace=False)
    lens[picks[0]] = 0
    if len(picks) > 1:
        lens[picks[1]] = max_len + 1 + int(rng.integers(0, 100))
    if len(picks) > 2:
        lens[picks[2]] = -7
    for r in picks[3:]:
        nb = -(-min(int(lens[r]), max_len) // 16)
        for j in {0, nb - 1, nb // 2}:
            tables[r, j] = [-1, nb_pool, 2**31 - 1][j % 3]
    say(f"check: seed {seed}, {rows} rows, stride {stride}, max_len {max_len}")
    pool, cache = _cache(torch, nb_pool)
    want = expected(tables, lens, max_len, nb_pool)
    assert want[0] >= 1
    assert _run(torch, cache, tables, lens, max_len) == want

    # the prefill contract: query ranges, with planted empty, too long and out-of-range rows
    n = np.minimum(rng.integers(1, 40, size=rows), np.maximum(lens, 1)).astype(np.int64)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    total_q = int(qs[-1])
    assert _run(torch, cache, tables, lens, max_len, qs, total_q) == expected(tables, lens, max_len, nb_pool, qs,
                                                                                total_q)
    qs2 = qs.copy()
    qs2[min(2, rows)] = qs2[min(2, rows) - 1]          # an empty row
    qs2[-1] = total_q + 5                               # past total_q
    want = expected(tables, lens, max_len, nb_pool, qs2, total_q)
    assert want[2] >= 1
    assert _run(torch, cache, tables, lens, max_len, qs2, total_q) == want


def test_report_overwritten_and_graph_replays():
    """The report is written whole by every call (nothing to clear), so a
    captured call replays correctly over inputs changed between replays."""
    torch = torch_cuda()
    rng = np.random.default_rng(9)
    rows, stride, nb_pool = 24, 64, 300
    max_len = stride * 16
    tables = rng.integers(0, nb_pool, size=(rows, stride)).astype(np.int32)
    lens = rng.integers(1, max_len + 1, size=rows).astype(np.int32)
    pool, cache = _cache(torch, nb_pool)
    t_d, l_d = dev(tables, torch), dev(lens, torch)
    report = torch.full((4,), -99, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        pkv.check_tables(cache, t_d, l_d, max_len, report)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.check_tables(cache, t_d, l_d, max_len, report)
    torch.cuda.synchronize()
    for i in range(4):
        t2, l2 = tables.copy(), lens.copy()
        if i % 2:
            l2[rng.integers(rows)] = 0
            t2[rng.integers(rows), 0] = -3
        t_d.copy_(dev(t2, torch))
        l_d.copy_(dev(l2, torch))
        report.fill_(777)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [int(x) for x in report.cpu().numpy()]
        say(f"replay {i}: {got}")
        assert got == expected(t2, l2, max_len, nb_pool)
