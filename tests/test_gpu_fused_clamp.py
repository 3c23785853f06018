"""The fused append + decode calls with a row longer than max_context_len and a
row of length 0.

Such rows break the call's length contract: they are read clamped (for memory
safety) and their output is unspecified, but they must append nothing -- the
long row's new token slot lies past the clamp, and writing the token anywhere
else would overwrite a cached token of that row; the empty row has no slot at
all.  Every other row appends and decodes as usual.  For the FP16 call, the grouped-query call (4 query heads per KV head)
and the 8-bit call: the pool (codes and scales) must equal the oracle's append
of the in-contract rows alone, byte for byte over the whole pool, and the
in-contract rows' outputs must match the oracle."""
import numpy as np
import pytest

import oracle.fp8 as ofp8
import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_f64, say, torch_cuda
from tests.tolerance import assert_close
from workloads import SCALE, build_batch

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

LENS = [40, 300, 601, 600, 17]  # row 2 ends one token past max_context_len
MAXL = 600
OVER = 2
EMPTY = 4  # passed to the call with context length 0
KEEP = [r for r in range(len(LENS)) if r not in (OVER, EMPTY)]


def _batch(heads, seed):
    return build_batch("fused-clamp", seed, LENS, [1] * len(LENS), num_blocks=sum(-(-L // 16) for L in LENS) + 6,
                       num_layers=2, num_heads=heads, stride=-(-max(LENS) // 16) + 2)


def _append_kept(b, layer):
    """The oracle's append of every row's new token except the over-long row's."""
    keep = np.array(KEEP)
    return opaged.append(b.pool, layer, b.k_new[layer][keep], b.v_new[layer][keep], b.positions[keep],
                         b.request_of_token[keep], b.block_tables)


@pytest.mark.parametrize("kind", ["fp16", "gqa4", "fp8"])
def test_fused_append_skips_row_past_max_context_len(kind):
    torch = torch_cuda()
    layer = 1
    G = 4 if kind == "gqa4" else 1
    Hkv = 8 if kind == "gqa4" else 32
    Hq = Hkv * G
    b = _batch(Hkv, 71 + G)
    R = len(LENS)
    rng = np.random.default_rng(90 + G)
    q = rng.standard_normal((R, Hq, 128), dtype=np.float32).astype(np.float16).view(np.uint16)
    lens_call = b.context_lens.copy()
    lens_call[EMPTY] = 0
    tables, lens_d = dev(b.block_tables, torch), dev(lens_call, torch)
    k, v = dev(b.k_new[layer], torch), dev(b.v_new[layer], torch)
    out = torch.empty((R, Hq, 128), dtype=torch.float16, device="cuda")
    say(f"fused append with row {OVER} at {LENS[OVER]} > max_context_len {MAXL} and row {EMPTY} empty ({kind})")
    want_pool = _append_kept(b, layer)
    if kind == "fp8":
        codes, scales = ofp8.quantize_rows(b.pool)
        codes_d = torch.from_numpy(codes).cuda()
        scales_d = torch.from_numpy(scales).cuda()
        cache = pkv.PagedCache8(codes_d, scales_d)
        ws = torch.empty(pkv.decode_workspace_size_fp8(cache, R, MAXL), dtype=torch.uint8, device="cuda")
        pkv.decode_attention_append_fp8(cache, layer, out, dev(q, torch), k, v, tables, lens_d, MAXL, SCALE, ws)
        torch.cuda.synchronize()
        keep = np.array(KEEP)
        want_c, want_s = ofp8.append(codes, scales, layer, b.k_new[layer][keep], b.v_new[layer][keep],
                                     b.positions[keep], b.request_of_token[keep], b.block_tables)
        assert np.array_equal(codes_d.cpu().numpy(), want_c), "8-bit codes differ from the in-contract append"
        assert np.array_equal(scales_d.cpu().numpy().view(np.uint32), want_s.view(np.uint32)), "8-bit scales differ"
        ref = ofp8.decode(want_c, want_s, layer, q[KEEP], b.block_tables[KEEP], b.context_lens[KEEP], SCALE)
    else:
        pool_d = dev(b.pool, torch)
        cache = pkv.PagedCache(pool_d)
        ws = torch.empty(pkv.decode_workspace_size_gqa(cache, Hq, R, MAXL), dtype=torch.uint8, device="cuda")
        if G == 1:
            pkv.decode_attention_append(cache, layer, out, dev(q, torch), k, v, tables, lens_d, MAXL, SCALE, ws)
        else:
            pkv.decode_attention_append_gqa(cache, Hq, layer, out, dev(q, torch), k, v, tables, lens_d, MAXL, SCALE,
                                            ws)
        torch.cuda.synchronize()
        got_pool = pool_d.cpu().numpy().view(np.uint16)
        assert np.array_equal(got_pool, want_pool), "pool differs from the in-contract rows' append"
        ref = opaged.decode(want_pool[:, layer], q[KEEP], b.block_tables[KEEP], b.context_lens[KEEP], SCALE, group=G)
    s = assert_close(host_f64(out.view(torch.int16))[KEEP], ref, f"{kind} in-contract rows")
    say(f"  {s}")
