"""8-bit KV cache on the GPU: quantizing append bit-exact against the oracle,
decode over the dequantized cache against the oracle, and the quality cost
against FP16 attention measured by context length."""
import numpy as np
import pytest

import oracle.fp8 as ofp8
import oracle.paged as opaged
import paged_kv_cache_pkv_amd as pkv
from tests.gpu_util import dev, host_f64, say, torch_cuda
from tests.tolerance import assert_close, compare
from workloads import SCALE, build_batch, c1_tiny

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def _random_cache(seed, shape):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, shape, dtype=np.uint8)
    scales = rng.standard_normal(shape[:5], dtype=np.float32)
    return codes, scales


def _quantized_pool(pool_bits):
    """Codes and scales of every (block, layer, kv, head, slot) row of an FP16 pool."""
    return ofp8.quantize_rows(pool_bits)


def _gpu_cache(torch, codes, scales):
    codes_d = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    scales_d = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    return pkv.PagedCache8(codes_d, scales_d), codes_d, scales_d


@pytest.mark.parametrize("which", ["tiny", "bulk"])
def test_append_fp8_bitexact(which):
    torch = torch_cuda()
    if which == "tiny":
        b = c1_tiny()
        layer = 0
    else:
        b = build_batch("fp8-bulk", 23, [700, 33, 16, 1], [512, 1, 1, 1], num_blocks=80, num_layers=3,
                        num_heads=32, stride=48)
        layer = 2
    shape = b.pool.shape
    codes, scales = _random_cache(5, shape)
    say(f"append fp8 {which}")
    cache, codes_d, scales_d = _gpu_cache(torch, codes, scales)
    pkv.append_fp8(cache, layer, dev(b.k_new[layer], torch), dev(b.v_new[layer], torch), dev(b.positions, torch),
                   dev(b.request_of_token, torch), dev(b.block_tables, torch))
    torch.cuda.synchronize()
    want_c, want_s = ofp8.append(codes, scales, layer, b.k_new[layer], b.v_new[layer], b.positions,
                                 b.request_of_token, b.block_tables)
    assert np.array_equal(codes_d.cpu().numpy(), want_c)
    assert np.array_equal(scales_d.cpu().numpy().view(np.uint32), want_s.view(np.uint32))


CASES = [
    # name, heads, layers, lens
    ("ragged", 32, 1, [1, 2, 15, 16, 17, 100, 255, 256, 257, 512]),
    # the edges of a wave's 128-token share and of a 512-token range
    ("share-edges", 8, 1, [127, 128, 129, 383, 384, 385, 511, 512, 513, 1024, 1025]),
    ("multi-split", 32, 2, [513, 1025, 2600]),
    ("odd-heads", 5, 1, [300, 1, 700]),
    # the most heads the library accepts
    ("max-heads", 128, 1, [300, 17]),
    # many rows of mixed lengths
    ("many-rows", 4, 1, [int(x) for x in np.random.default_rng(81).integers(1, 900, 500)]),
]


@pytest.mark.parametrize("name,heads,layers,lens", CASES, ids=[c[0] for c in CASES])
def test_decode_fp8_parity(name, heads, layers, lens):
    torch = torch_cuda()
    b = build_batch(f"fp8-{name}", 31, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 4,
                    num_layers=layers, num_heads=heads, stride=max(-(-L // 16) for L in lens))
    pool = b.pool
    for layer in range(layers):
        pool = opaged.append(pool, layer, b.k_new[layer], b.v_new[layer], b.positions, b.request_of_token,
                             b.block_tables)
    codes, scales = _quantized_pool(pool)  # poisoned slots quantize to junk the kernel must never read
    cache, _, _ = _gpu_cache(torch, codes, scales)
    R = len(lens)
    maxL = max(lens)
    ws = torch.empty(max(pkv.decode_workspace_size_fp8(cache, R, maxL), 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
    for layer in range(layers):
        say(f"decode fp8 {name} heads={heads} layer {layer}")
        pkv.decode_attention_fp8(cache, layer, out, dev(b.q[layer], torch), dev(b.block_tables, torch),
                                 dev(b.context_lens, torch), maxL, SCALE, ws)
        torch.cuda.synchronize()
        ref = ofp8.decode(codes, scales, layer, b.q[layer], b.block_tables, b.context_lens, SCALE)
        assert_close(host_f64(out), ref, f"{name} layer {layer}")


def test_decode_fp8_beyond_64_ranges():
    """Rows of 79 and 66 ranges of 512 tokens: the 8-bit merge takes its ranges in several passes of 64."""
    torch = torch_cuda()
    lens = [40000, 33300, 300]
    b = build_batch("fp8-long", 33, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 4,
                    num_layers=1, num_heads=2, stride=max(-(-L // 16) for L in lens))
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    codes, scales = _quantized_pool(pool)
    cache, _, _ = _gpu_cache(torch, codes, scales)
    ws = torch.empty(pkv.decode_workspace_size_fp8(cache, len(lens), max(lens)), dtype=torch.uint8, device="cuda")
    out = torch.empty((len(lens), 2, 128), dtype=torch.float16, device="cuda")
    say(f"decode fp8 beyond 64 ranges lens={lens}")
    pkv.decode_attention_fp8(cache, 0, out, dev(b.q[0], torch), dev(b.block_tables, torch),
                             dev(b.context_lens, torch), max(lens), SCALE, ws)
    torch.cuda.synchronize()
    ref = ofp8.decode(codes, scales, 0, b.q[0], b.block_tables, b.context_lens, SCALE)
    assert_close(host_f64(out), ref, "fp8 beyond 64 ranges")


def test_fp8_append_then_decode():
    """End to end: the library quantizes the step's tokens, then decode reads
    them (each row attends over its own new token)."""
    torch = torch_cuda()
    b = build_batch("fp8-e2e", 37, [40, 300, 1100], [1, 1, 1], num_blocks=100, num_layers=1, num_heads=32, stride=72)
    codes, scales = _quantized_pool(b.pool)
    cache, codes_d, scales_d = _gpu_cache(torch, codes, scales)
    tabs = dev(b.block_tables, torch)
    pkv.append_fp8(cache, 0, dev(b.k_new[0], torch), dev(b.v_new[0], torch), dev(b.positions, torch),
                   dev(b.request_of_token, torch), tabs)
    ws = torch.empty(pkv.decode_workspace_size_fp8(cache, 3, 1100), dtype=torch.uint8, device="cuda")
    out = torch.empty((3, 32, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_fp8(cache, 0, out, dev(b.q[0], torch), tabs, dev(b.context_lens, torch), 1100, SCALE, ws)
    torch.cuda.synchronize()
    want_c, want_s = ofp8.append(codes, scales, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token,
                                 b.block_tables)
    assert np.array_equal(codes_d.cpu().numpy(), want_c)
    ref = ofp8.decode(want_c, want_s, 0, b.q[0], b.block_tables, b.context_lens, SCALE)
    assert_close(host_f64(out), ref, "append then decode")


def test_fp8_quality_against_fp16():
    """The quality cost of the 8-bit cache: FP8 decode against FP16-cache
    attention (the oracle over the original values), by context length.
    Printed for the record; the bound only guards against a broken path."""
    torch = torch_cuda()
    lens = [256, 2048, 8192]
    b = build_batch("fp8-quality", 41, lens, [1, 1, 1], num_blocks=sum(L // 16 for L in lens) + 4, num_layers=1,
                    num_heads=32, stride=512, poison=False)
    pool = opaged.append(b.pool, 0, b.k_new[0], b.v_new[0], b.positions, b.request_of_token, b.block_tables)
    codes, scales = _quantized_pool(pool)
    cache, _, _ = _gpu_cache(torch, codes, scales)
    ws = torch.empty(pkv.decode_workspace_size_fp8(cache, 3, 8192), dtype=torch.uint8, device="cuda")
    out = torch.empty((3, 32, 128), dtype=torch.float16, device="cuda")
    pkv.decode_attention_fp8(cache, 0, out, dev(b.q[0], torch), dev(b.block_tables, torch),
                             dev(b.context_lens, torch), 8192, SCALE, ws)
    torch.cuda.synchronize()
    got = host_f64(out)
    ref16 = opaged.decode(pool[:, 0], b.q[0], b.block_tables, b.context_lens, SCALE)
    for r, L in enumerate(lens):
        s = compare(got[r], ref16[r])
        say(f"fp8 vs fp16 attention, context {L}: max_abs {s['max_abs']:.2e}, rms {np.sqrt(np.mean((got[r] - ref16[r]) ** 2)):.2e}")
        assert s["max_abs"] < 0.05


@pytest.mark.parametrize("heads", [32, 5])
def test_fp8_appending_decode_equals_append_then_decode_bitwise(heads):
    """pkv_decode_attention_append_fp8 leaves the same codes and scales and the
    same output bits as pkv_append_fp8 followed by pkv_decode_attention_fp8
    (5 heads: a workgroup whose last waves hold no head)."""
    torch = torch_cuda()
    lens = [1, 4, 5, 16, 17, 255, 256, 257, 700, 2600]
    b = build_batch("fp8-fused", 39, lens, [1] * len(lens), num_blocks=sum(-(-L // 16) for L in lens) + 6,
                    num_layers=2, num_heads=heads, stride=max(-(-L // 16) for L in lens) + 2)
    codes, scales = _quantized_pool(b.pool)
    layer = 1
    R, maxL = len(lens), max(lens)
    say(f"fp8 appending decode vs append + decode, lens={lens}")

    def run(fused):
        cache, codes_d, scales_d = _gpu_cache(torch, codes, scales)
        ws = torch.empty(pkv.decode_workspace_size_fp8(cache, R, maxL), dtype=torch.uint8, device="cuda")
        out = torch.empty((R, heads, 128), dtype=torch.float16, device="cuda")
        tabs, lens_d = dev(b.block_tables, torch), dev(b.context_lens, torch)
        k, v = dev(b.k_new[layer], torch), dev(b.v_new[layer], torch)
        if fused:
            pkv.decode_attention_append_fp8(cache, layer, out, dev(b.q[layer], torch), k, v, tabs, lens_d, maxL,
                                            SCALE, ws)
        else:
            pkv.append_fp8(cache, layer, k, v, dev(b.positions, torch), dev(b.request_of_token, torch), tabs)
            pkv.decode_attention_fp8(cache, layer, out, dev(b.q[layer], torch), tabs, lens_d, maxL, SCALE, ws)
        torch.cuda.synchronize()
        return (codes_d.cpu().numpy(), scales_d.cpu().numpy().view(np.uint32), out.cpu().numpy().view(np.uint16))

    ca, sa, oa = run(False)
    cb, sb, ob = run(True)
    assert np.array_equal(ca, cb), "fused 8-bit append codes differ"
    assert np.array_equal(sa, sb), "fused 8-bit append scales differ"
    assert np.array_equal(oa, ob), "fused 8-bit decode differs from append + decode"
