"""pkv_decode_attention_append_noalloc (the call for callers that cannot
allocate) against pkv_decode_attention_append with a caller workspace: the
same pool bytes and the same output bits, on two calls in a row, the second
with a smaller batch, so that whatever the first call left in the library's
scratch array cannot reach the second call's result.  Also: a call needing
more scratch than the array holds is refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, say, torch_cuda
from workloads import SCALE, build_batch

pytestmark = pytest.mark.gpu


def _run(torch, b, layer, noalloc):
    pool_d = dev(b.pool, torch)
    cache = pkv.PagedCache(pool_d)
    R, maxL = b.rows, int(b.context_lens.max())
    out = torch.empty((R, b.num_heads, 128), dtype=torch.float16, device="cuda")
    args = (cache, layer, out, dev(b.q[layer], torch), dev(b.k_new[layer], torch), dev(b.v_new[layer], torch),
            dev(b.block_tables, torch), dev(b.context_lens, torch), maxL, SCALE)
    if noalloc:
        pkv.decode_attention_append_noalloc(*args)
    else:
        ws = torch.empty(max(pkv.decode_workspace_size(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
        pkv.decode_attention_append(*args, ws)
    torch.cuda.synchronize()
    return pool_d.cpu().numpy().view(np.uint16), out.cpu().numpy().view(np.uint16)


def test_noalloc_equals_workspace_call_twice():
    torch = torch_cuda()
    big = [5000, 4097, 300, 2600, 1, 17, 3000, 256, 257, 1600, 4500, 800]
    small = [900, 40, 513, 2]
    for i, lens in enumerate((big, small)):
        b = build_batch(f"noalloc-{i}", 81 + i, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 8,
                        num_layers=2, stride=-(-max(lens) // 16) + 2)
        say(f"no-alloc call {i}: {len(lens)} rows, contexts up to {max(lens)}")
        want_pool, want_out = _run(torch, b, 1, noalloc=False)
        got_pool, got_out = _run(torch, b, 1, noalloc=True)
        assert np.array_equal(got_pool, want_pool), f"call {i}: pool bytes differ"
        assert np.array_equal(got_out, want_out), f"call {i}: output bits differ"


def test_noalloc_refuses_more_than_its_scratch():
    torch = torch_cuda()
    L = pkv.lib()
    d = pkv._lib.PkvCacheDesc(ctypes.c_void_p(0x100000), 64, 1, 128, 16, 128)
    fake = ctypes.c_void_p(0x200000)
    # 128 heads x 64 rows x 64 ranges of 520 bytes: 272 MB of partials
    rc = L.pkv_decode_attention_append_noalloc(ctypes.byref(d), 0, fake, fake, fake, fake, fake, 1024, fake, 64,
                                               16384, 0.088, None)
    assert rc == -6 and b"at most" in L.pkv_last_error()
    assert torch.cuda.is_available()
