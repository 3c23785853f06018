"""Continuous-batching trace on the GPU at a small size: rows join and leave
every step, long prompts share ref-counted prefix blocks, tables grow through
the library's block pool.  Decode outputs of sampled steps are checked against
the fp64 oracle, which rebuilds every row's context from the seeded draws (and
the prefix blocks' initial contents) without reading anything the kernels
wrote; pool invariants are checked every step and after the drain.  The full
size runs in test_gpu_trace_full.py."""
import pytest

from tests.gpu_util import say, torch_cuda
from tests.trace_check import TraceChecker

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shared_decode", [False, True], ids=["plain-decode", "shared-prefix-decode"])
def test_trace_parity_and_pool_invariants(shared_decode):
    torch = torch_cuda()
    from paged_kv_cache_pkv_amd.trace import ContinuousBatchTrace

    NB = 3000
    tr = ContinuousBatchTrace(torch, seed=11, num_blocks=NB, max_rows=8, prefix_tokens=512, prompt_range=(50, 1400),
                              answer_range=(1, 40), heads=32, shared_decode=shared_decode)
    chk = TraceChecker(tr)
    npre = len(tr.prefix_ids)
    for s in range(60):
        snap = tr.step()
        chk.record(snap)
        # pool invariants: prefix held once by the trace plus once per sharing row
        sharers = sum(1 for r in tr.rows if r.shared)
        for b in tr.prefix_ids:
            assert tr.pool.ref_count(int(b)) == 1 + sharers
        held = sum(r.nblk - r.shared // 16 for r in tr.rows)
        assert tr.pool.num_free + held + npre == NB
        if s % 7 == 3:
            say(f"trace step {s} (shared_decode={shared_decode}): rows {len(snap['reqs'])} lens {list(snap['lens'])}")
            chk.keep(snap)
    assert tr.next_req > 8  # rows left and were refilled
    tr.drain()
    assert tr.pool.num_free == NB
    assert all(tr.pool.ref_count(b) == 0 for b in range(NB))
    tot = chk.check()
    say(f"trace parity: {tot}")
    assert tot["rows"] >= 40
    assert tot["bad"] == 0 and tot["nan"] == 0, tot
