"""8-bit KV cache: FP8 codes with one scale per (token, head).  NumPy on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

An 8-bit cache halves the bytes of every cached token and so the attention
read traffic, with a quality risk that grows with context length (Inference
Infrastructure, seeitflow.com, its paragraph on KV-cache precision; The inference engine,
wpnews.pro, "IO-aware attention and quantization attack different costs":
KV quantization changes bytes per token but adds accuracy questions).  The
pages fix no format; the reading taken (one fp32 scale per row of 128 values,
E4M3 codes) is written out here by its definition:

* Codes are FP8 E4M3 ("E4M3FN" of the OCP 8-bit floating point format): one
  sign bit, four exponent bits with bias 7, three mantissa bits; exponent 0 is
  subnormal (m / 8 * 2^-6), code 0x7F / 0xFF is NaN and there is no infinity,
  so the largest finite magnitude is 1.75 * 2^8 = 448.
* Every (token, head) row of 128 values x gets the scale s = amax / 448 with
  amax = max |x|; the code of x is the finite E4M3 value nearest to
  x * (448 / amax) (that product taken in fp32), a tie between two neighbours
  going to the one with the even mantissa, and magnitudes above 448 saturating
  to 448.  A zero row has s = 0 and all-zero codes.
* A cached value reads back as decode(code) * s.

Pool arrays: codes [num_blocks, layers, 2, heads, 16, head_dim] uint8 and
scales [num_blocks, layers, 2, heads, 16] float32, key first (index 0) and
value second, as in the FP16 pool.
"""
from __future__ import annotations

import numpy as np

from . import paged

FP8_MAX = 448.0


def decode_table() -> np.ndarray:
    """The value of every E4M3 code, float64 [256] (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def encode(x) -> np.ndarray:
    """E4M3 code of each float32 value, by the definition: the finite value of
    the format nearest to |x| (the 127 non-negative codes 0x00..0x7E, whose
    values increase with the code), a tie between two neighbours going to the
    even code (the code's low bit is the mantissa's last bit), magnitudes above
    448 saturating to 448 (0x7E); the sign bit is x's.  Returns uint8."""
    x = np.asarray(x, dtype=np.float32)
    sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
    a = np.abs(x).astype(np.float64)  # exact: float32 values are float64 values
    vals = decode_table()[:0x7F]      # non-negative finite values, increasing with the code
    hi = np.clip(np.searchsorted(vals, a, side="left"), 1, 0x7E)  # vals[hi-1] < a <= vals[hi], clipped
    lo = hi - 1
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= FP8_MAX, 0x7E, code)  # saturation (also the clipped search past 448)
    code = np.where(a <= vals[0], 0, code)     # zero
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_rows(x_bits):
    """FP16 bit rows [..., 128] -> (codes uint8 [..., 128], scales float32 [...]).

    s = amax / 448; codes = encode(x * (448 / amax)); a zero row gives s = 0."""
    x = np.asarray(x_bits).view(np.float16).astype(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    inv = (np.float32(FP8_MAX) / safe).astype(np.float32)
    scaled = (x * inv[..., None]).astype(np.float32)
    codes = encode(scaled)
    codes = np.where((amax > 0)[..., None], codes, np.uint8(0)).astype(np.uint8)
    scales = np.where(amax > 0, (amax / np.float32(FP8_MAX)).astype(np.float32), np.float32(0.0))
    return codes, scales.astype(np.float32)


def dequantize(codes, scales) -> np.ndarray:
    """Cached values as float64: decode(code) * scale."""
    return decode_table()[np.asarray(codes)] * np.asarray(scales, dtype=np.float64)[..., None]


def append(codes_pool, scales_pool, layer, k_new, v_new, positions, request_of_token, block_tables):
    """Quantize each new token's keys and values per head and write codes and
    scales into its block slot (the FP16 append's placement, paged.locate).
    Returns new (codes_pool, scales_pool)."""
    cp = codes_pool.copy()
    sp = scales_pool.copy()
    kc, ks = quantize_rows(k_new)
    vc, vs = quantize_rows(v_new)
    for t in range(len(positions)):
        b, s = paged.locate(block_tables[int(request_of_token[t])], int(positions[t]))
        cp[b, layer, 0, :, s, :] = kc[t]
        cp[b, layer, 1, :, s, :] = vc[t]
        sp[b, layer, 0, :, s] = ks[t]
        sp[b, layer, 1, :, s] = vs[t]
    return cp, sp


class _Dequantized:
    """pool_layer view for paged.gather_kv: block id -> [2, heads, 16, head_dim]
    FP16-free float values, decoded on access."""

    def __init__(self, codes_layer, scales_layer):
        self.c = codes_layer
        self.s = scales_layer

    def __getitem__(self, b):
        return dequantize(self.c[b], self.s[b])


def gather_kv(codes_pool, scales_pool, layer, table_row, seq_len):
    """Contiguous dequantized K and V of one row, float64 [heads, L, head_dim]."""
    return _gather_float(_Dequantized(codes_pool[:, layer], scales_pool[:, layer]), table_row, seq_len)


def _gather_float(pool_layer, table_row, seq_len, block_size=16):
    full = seq_len // block_size
    parts_k, parts_v = [], []
    for j in range(full):
        blk = pool_layer[int(table_row[j])]
        parts_k.append(blk[0])
        parts_v.append(blk[1])
    rem = seq_len - full * block_size
    if rem:
        blk = pool_layer[int(table_row[full])]
        parts_k.append(blk[0][:, :rem])
        parts_v.append(blk[1][:, :rem])
    return np.concatenate(parts_k, axis=1), np.concatenate(parts_v, axis=1)


def decode(codes_pool, scales_pool, layer, q, block_tables, context_lens, scale):
    """Decode attention over the dequantized cache (one query per row at position
    context_lens[r] - 1), float64 [R, heads, head_dim]."""
    outs = []
    for r in range(len(context_lens)):
        L = int(context_lens[r])
        K, V = gather_kv(codes_pool, scales_pool, layer, block_tables[r], L)
        outs.append(paged.attention(np.asarray(q)[r:r + 1], K, V, [L - 1], scale)[0])
    return np.stack(outs)
