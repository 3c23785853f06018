"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin fails for each.  This shows the pins constrain every part of the
oracle rather than restating it."""
import numpy as np
import pytest

import oracle.blocks as oblocks
import oracle.fp8 as ofp8
import oracle.paged as paged
import oracle.pool as opool
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_attention = paged.attention
_gather = paged.gather_kv
_locate = paged.locate


def _attn_no_scale(q, K, V, pos, scale):
    return _attention(q, K, V, pos, 1.0)


def _attn_swap_kv(q, K, V, pos, scale):
    return _attention(q, V, K, pos, scale)


def _attn_hide_own(q, K, V, pos, scale):
    pos = np.asarray(pos)
    if np.all(pos >= 1):
        return _attention(q, K, V, pos - 1, scale)
    return _attention(q, K, V, pos, scale)


def _attn_neg_sign(q, K, V, pos, scale):
    return _attention(q, K, V, pos, -scale)


def _gather_reverse_slots(pool_layer, row, L, block_size=16):
    K, V = _gather(pool_layer, row, L, block_size)
    if L >= 2:
        K = K.copy(); V = V.copy()
        K[:, :2] = K[:, 1::-1]
        V[:, :2] = V[:, 1::-1]
    return K, V


def _gather_drop_tail(pool_layer, row, L, block_size=16):
    full = (L // block_size) * block_size
    if full and full != L:
        K, V = _gather(pool_layer, row, full, block_size)
        K2, V2 = _gather(pool_layer, row, L, block_size)
        K2 = K2.copy(); V2 = V2.copy()
        K2[:, full:] = K[:, -1:]
        V2[:, full:] = V[:, -1:]
        return K2, V2
    return _gather(pool_layer, row, L, block_size)


def _locate_swapped(row, position, block_size=16):
    return int(row[position % block_size if position % block_size < len(row) else 0]), position // block_size % block_size


def _group_kv_tiled(K, V, group):
    if group == 1:
        return K, V
    return np.tile(K, (group, 1, 1)), np.tile(V, (group, 1, 1))


_chunked = paged.chunked_prefill


def _chunk_positions_late(pool_layer, q, query_start, block_tables, context_lens, scale, rows=None, group=1):
    """Each chunk query placed one position later: it sees one key past its own."""
    qs = np.asarray(query_start)
    outs = []
    for r in (range(len(context_lens)) if rows is None else rows):
        L = int(context_lens[r])
        a, b = int(qs[r]), int(qs[r + 1])
        K, V = paged.group_kv(*paged.gather_kv(pool_layer, block_tables[r], L), group)
        pos = np.minimum(np.arange(L - (b - a), L) + 1, L - 1)
        outs.append(paged.attention(np.asarray(q)[a:b], K, V, pos, scale))
    return np.concatenate(outs, axis=0)


def _chunk_first_query_shifted(pool_layer, q, query_start, block_tables, context_lens, scale, rows=None, group=1):
    """The row's queries read one slot late in the flat token list (off-by-one on query_start)."""
    qs = np.asarray(query_start).copy()
    qs[1:-1] += 1
    qs = np.minimum(qs, len(q))
    return _chunked(pool_layer, q, qs, block_tables, context_lens, scale, rows, group) if np.all(np.diff(qs) >= 1) \
        else _chunked(pool_layer, np.roll(q, 1, axis=0), query_start, block_tables, context_lens, scale, rows, group)


def _decode_drops_last(pool_layer, q, block_tables, context_lens, scale, rows=None, group=1):
    """Decode over one token fewer than the row holds (the appended token left out)."""
    lens = np.maximum(np.asarray(context_lens) - 1, 1)
    rows = range(len(context_lens)) if rows is None else rows
    outs = []
    for r in rows:
        L = int(lens[r])
        K, V = paged.group_kv(*paged.gather_kv(pool_layer, block_tables[r], L), group)
        outs.append(paged.attention(np.asarray(q)[r:r + 1], K, V, [L - 1], scale)[0])
    return np.stack(outs)


def _blocks_floor(n, block_size=16):
    return int(n) // block_size


MUTANTS = [
    ("attention", _attn_no_scale),
    ("attention", _attn_swap_kv),
    ("attention", _attn_hide_own),
    ("attention", _attn_neg_sign),
    ("gather_kv", _gather_reverse_slots),
    ("gather_kv", _gather_drop_tail),
    ("locate", _locate_swapped),
    ("group_kv", _group_kv_tiled),
    ("chunked_prefill", _chunk_positions_late),
    ("chunked_prefill", _chunk_first_query_shifted),
    ("decode", _decode_drops_last),
]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[f"{n}:{f.__name__}" for n, f in MUTANTS])
def test_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(paged, name, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {fn.__name__}"


def test_pool_mutant_is_caught(monkeypatch):
    monkeypatch.setattr(opool, "blocks_needed", _blocks_floor)
    with pytest.raises(AssertionError):
        oracle_pins.pin_block_arithmetic()


_copy_blocks = oblocks.copy_blocks
_swap_in = oblocks.swap_in


def _copy_first_layer_only(pool, src, dst):
    out = _copy_blocks(pool, src, dst)
    for d in np.asarray(dst).tolist():
        out[d, 1:] = pool[d, 1:]
    return out


def _copy_wrong_direction(pool, src, dst):
    return _copy_blocks(pool, dst, src)


def _swap_in_reversed(pool, host, ids):
    return _swap_in(pool, host, list(ids)[::-1])


@pytest.mark.parametrize("name,fn", [("copy_blocks", _copy_first_layer_only), ("copy_blocks", _copy_wrong_direction),
                                     ("swap_in", _swap_in_reversed)],
                         ids=["copy_first_layer_only", "copy_wrong_direction", "swap_in_reversed"])
def test_blocks_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oblocks, name, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {fn.__name__}"


_encode = ofp8.encode
_quantize_rows = ofp8.quantize_rows


def _encode_round_half_up(x):
    x = np.asarray(x, dtype=np.float32)
    nudged = np.where(np.abs(x) > 0, x * np.float32(1 + 2.0 ** -20), x).astype(np.float32)
    return _encode(nudged)


def _quantize_wrong_scale(x_bits):
    codes, sc = _quantize_rows(x_bits)
    return codes, (sc * np.float32(448.0 / 447.0)).astype(np.float32)


@pytest.mark.parametrize("name,fn", [("encode", _encode_round_half_up), ("quantize_rows", _quantize_wrong_scale)],
                         ids=["encode_round_half_up", "quantize_wrong_scale"])
def test_fp8_mutant_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(ofp8, name, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {fn.__name__}"
