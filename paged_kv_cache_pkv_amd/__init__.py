"""Paged KV-cache attention for MI355X: Python binding of libpkv.so.

Argument marshalling only.  Every step of the path runs in the library: the
host block pool in C++, append / decode / chunked prefill in gfx950 HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  If the
library is missing, calls raise; nothing falls back to another
implementation.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

BLOCK_SIZE = 16
HEAD_DIM = 128

PKV_OK = 0
ERRORS = {-1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "OUT_OF_BLOCKS", -4: "DOUBLE_FREE", -5: "BAD_BLOCK",
          -6: "WORKSPACE", -7: "HIP"}


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


def lib():
    return _lib.load()


def _check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, lib().pkv_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(_lib.c_i32_p)


def version() -> str:
    return lib().pkv_version().decode()


def blocks_needed(num_tokens: int) -> int:
    return int(lib().pkv_blocks_needed(int(num_tokens)))


def split_tokens() -> int:
    return int(lib().pkv_split_tokens())


class BlockPool:
    """Host block pool (free list + reference counts) owned by libpkv."""

    def __init__(self, num_blocks: int, free_list=None):
        self._h = ctypes.c_void_p()
        if free_list is None:
            _check(lib().pkv_pool_create(int(num_blocks), ctypes.byref(self._h)))
        else:
            fl = _i32(free_list)
            _check(lib().pkv_pool_create_from_list(int(num_blocks), _iptr(fl), fl.size, ctypes.byref(self._h)))

    def close(self):
        if self._h:
            lib().pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(max(int(n), 0), dtype=np.int32)
        _check(lib().pkv_alloc(self._h, int(n), _iptr(out)))
        return out

    def ref(self, ids) -> None:
        a = _i32(ids)
        _check(lib().pkv_ref(self._h, _iptr(a), a.size))

    def free(self, ids) -> None:
        a = _i32(ids)
        _check(lib().pkv_free(self._h, _iptr(a), a.size))

    def grow(self, table: np.ndarray, length: int, num_tokens: int) -> int:
        """Grow int32 `table` (its first `length` entries in use) to cover
        num_tokens; returns the new length.  Raises PkvError(OUT_OF_BLOCKS)
        with no change when the free list is short."""
        if table.dtype != np.int32 or not table.flags.c_contiguous:
            raise TypeError("table must be a C-contiguous int32 array")
        n = ctypes.c_int32(int(length))
        _check(lib().pkv_grow(self._h, _iptr(table), ctypes.byref(n), table.size, int(num_tokens)))
        return int(n.value)

    def grow_rows(self, tables: np.ndarray, table_lens: np.ndarray, num_tokens) -> int:
        """Grow every row r of int32 `tables` [R, stride] (its first table_lens[r]
        entries in use, updated in place) to cover num_tokens[r] tokens, rows in
        order, in one library call.  Returns the number of rows grown: R, or the
        index of the first row the free list could not cover (that row and the
        later ones are unchanged)."""
        for a, what in ((tables, "tables"), (table_lens, "table_lens")):
            if a.dtype != np.int32 or not a.flags.c_contiguous:
                raise TypeError(f"{what} must be a C-contiguous int32 array")
        R, stride = tables.shape
        if table_lens.shape != (R,):
            raise ValueError("table_lens must hold one length per row")
        need = _i32(num_tokens)
        if need.shape != (R,):
            raise ValueError("num_tokens must hold one count per row")
        done = ctypes.c_int32(0)
        rc = lib().pkv_grow_rows(self._h, _iptr(tables), int(stride), _iptr(table_lens), _iptr(need), int(R),
                                 ctypes.byref(done))
        if rc != PKV_OK and rc != -3:
            _check(rc)
        return int(done.value)

    @property
    def num_free(self) -> int:
        return int(lib().pkv_num_free(self._h))

    @property
    def num_blocks(self) -> int:
        return int(lib().pkv_num_blocks(self._h))

    def ref_count(self, block_id: int) -> int:
        return int(lib().pkv_ref_count(self._h, int(block_id)))

    def free_list(self) -> np.ndarray:
        n = lib().pkv_free_list(self._h, None, 0)
        out = np.empty(n, dtype=np.int32)
        lib().pkv_free_list(self._h, _iptr(out), n)
        return out


# ------------------------------------------------------------------ device side

def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dptr(t, what: str, dtype_bytes: int | None = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype_bytes is not None and t.element_size() != dtype_bytes:
        raise ValueError(f"{what} must have {dtype_bytes}-byte elements")
    return ctypes.c_void_p(t.data_ptr())


def _rows_need(rows: int, heads: int, **tensors):
    for what, t in tensors.items():
        _need(t, rows * heads * HEAD_DIM, what)


def _need(t, n: int, what: str):
    """The kernels index these arrays by the call's counts; a shorter tensor
    would be read or written past its end, so it is refused here."""
    if t is not None and int(t.numel()) < int(n):
        raise ValueError(f"{what} has {int(t.numel())} elements, the call needs {int(n)}")


class PagedCache:
    """Descriptor of a caller-owned device KV pool tensor
    [num_blocks, num_layers, 2, num_heads, 16, 128] of FP16 (or its uint16 bits)."""

    def __init__(self, pool):
        if pool.dim() != 6 or pool.shape[2] != 2 or pool.shape[4] != BLOCK_SIZE or pool.shape[5] != HEAD_DIM:
            raise ValueError("pool must be [num_blocks, num_layers, 2, num_heads, 16, 128]")
        _dptr(pool, "pool", 2)
        self.pool = pool
        nb, nl, _, nh, bs, hd = (int(x) for x in pool.shape)
        self.desc = _lib.PkvCacheDesc(ctypes.c_void_p(pool.data_ptr()), nb, nl, nh, bs, hd)

    @property
    def num_heads(self) -> int:
        return int(self.desc.num_heads)


def append(cache: PagedCache, layer: int, k_new, v_new, positions, request_of_token, block_tables, stream=None):
    T = int(positions.numel())
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(T, cache.num_heads, k_new=k_new, v_new=v_new)
    _need(request_of_token, T, "request_of_token")
    _check(lib().pkv_append(ctypes.byref(cache.desc), int(layer), _dptr(k_new, "k_new", 2), _dptr(v_new, "v_new", 2),
                            _dptr(positions, "positions", 4), _dptr(request_of_token, "request_of_token", 4), T,
                            _dptr(block_tables, "block_tables", 4), R, stride, _stream_ptr(stream)))


def decode_workspace_size(cache: PagedCache, num_rows: int, max_context_len: int) -> int:
    return int(lib().pkv_decode_workspace_size(ctypes.byref(cache.desc), int(num_rows), int(max_context_len)))


def decode_workspace_size_gqa(cache: PagedCache, num_q_heads: int, num_rows: int, max_context_len: int) -> int:
    return int(lib().pkv_decode_workspace_size_gqa(ctypes.byref(cache.desc), int(num_q_heads), int(num_rows),
                                                   int(max_context_len)))


def decode_attention(cache: PagedCache, layer: int, out, q, block_tables, context_lens, max_context_len: int,
                     scale: float, workspace=None, stream=None):
    decode_attention_gqa(cache, cache.num_heads, layer, out, q, block_tables, context_lens, max_context_len, scale,
                         workspace, stream)


def decode_attention_gqa(cache: PagedCache, num_q_heads: int, layer: int, out, q, block_tables, context_lens,
                         max_context_len: int, scale: float, workspace=None, stream=None):
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, num_q_heads, out=out, q=q)
    _need(context_lens, R, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (int(layer), _dptr(out, "out", 2), _dptr(q, "q", 2), _dptr(block_tables, "block_tables", 4), stride,
            _dptr(context_lens, "context_lens", 4), R, int(max_context_len), float(scale),
            _dptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream))
    if int(num_q_heads) == cache.num_heads:  # one query head per KV head: the plain call
        _check(lib().pkv_decode_attention(ctypes.byref(cache.desc), *args))
    else:
        _check(lib().pkv_decode_attention_gqa(ctypes.byref(cache.desc), int(num_q_heads), *args))


def decode_attention_append(cache: PagedCache, layer: int, out, q, k_new, v_new, block_tables, context_lens,
                            max_context_len: int, scale: float, workspace=None, stream=None):
    """Append each row's new token at position context_lens[r] - 1, then decode (one fused launch)."""
    decode_attention_append_gqa(cache, cache.num_heads, layer, out, q, k_new, v_new, block_tables, context_lens,
                                max_context_len, scale, workspace, stream)


def decode_attention_append_gqa(cache: PagedCache, num_q_heads: int, layer: int, out, q, k_new, v_new, block_tables,
                                context_lens, max_context_len: int, scale: float, workspace=None, stream=None):
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, num_q_heads, out=out, q=q)
    _rows_need(R, cache.num_heads, k_new=k_new, v_new=v_new)
    _need(context_lens, R, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (int(layer), _dptr(out, "out", 2), _dptr(q, "q", 2), _dptr(k_new, "k_new", 2), _dptr(v_new, "v_new", 2),
            _dptr(block_tables, "block_tables", 4), stride, _dptr(context_lens, "context_lens", 4), R,
            int(max_context_len), float(scale), _dptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream))
    if int(num_q_heads) == cache.num_heads:  # one query head per KV head: the plain call
        _check(lib().pkv_decode_attention_append(ctypes.byref(cache.desc), *args))
    else:
        _check(lib().pkv_decode_attention_append_gqa(ctypes.byref(cache.desc), int(num_q_heads), *args))


def decode_attention_append_noalloc(cache: PagedCache, layer: int, out, q, k_new, v_new, block_tables, context_lens,
                                    max_context_len: int, scale: float, stream=None):
    """decode_attention_append with the split-K partials in the library's own
    per-GPU scratch array (no workspace, no allocation); calls overlapping on
    one GPU race."""
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, cache.num_heads, out=out, q=q, k_new=k_new, v_new=v_new)
    _need(context_lens, R, "context_lens")
    _check(lib().pkv_decode_attention_append_noalloc(
        ctypes.byref(cache.desc), int(layer), _dptr(out, "out", 2), _dptr(q, "q", 2), _dptr(k_new, "k_new", 2),
        _dptr(v_new, "v_new", 2), _dptr(block_tables, "block_tables", 4), stride,
        _dptr(context_lens, "context_lens", 4), R, int(max_context_len), float(scale), _stream_ptr(stream)))


def decode_workspace_size_prefix(cache: PagedCache, num_rows: int, max_context_len: int, prefix_blocks: int) -> int:
    return int(lib().pkv_decode_workspace_size_prefix(ctypes.byref(cache.desc), int(num_rows), int(max_context_len),
                                                      int(prefix_blocks)))


def decode_attention_prefix(cache: PagedCache, layer: int, out, q, block_tables, context_lens, max_context_len: int,
                            scale: float, shares_prefix, prefix_blocks: int, workspace=None, stream=None):
    """Decode attention that reads a shared prefix of `prefix_blocks` blocks once
    for every row marked in `shares_prefix` (device int32 [rows])."""
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, cache.num_heads, out=out, q=q)
    _need(context_lens, R, "context_lens")
    _need(shares_prefix, R, "shares_prefix")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_attention_prefix(ctypes.byref(cache.desc), int(layer), _dptr(out, "out", 2),
                                             _dptr(q, "q", 2), _dptr(block_tables, "block_tables", 4), stride,
                                             _dptr(context_lens, "context_lens", 4), R, int(max_context_len),
                                             float(scale), _dptr(shares_prefix, "shares_prefix", 4),
                                             int(prefix_blocks), _dptr(workspace, "workspace"), ws_bytes,
                                             _stream_ptr(stream)))


def check_tables(cache: PagedCache, block_tables, context_lens, max_context_len: int, report, query_start=None,
                 total_q: int = 0, stream=None):
    """Count on the device the table entries, lengths and (with `query_start`)
    query ranges that break the calls' contract; `report` (device int32 [4])
    receives [bad lengths, bad table entries, bad query ranges, first bad row
    or -1].  Asynchronous: read `report` after the stream reaches it."""
    R, stride = (int(x) for x in block_tables.shape)
    _need(context_lens, R, "context_lens")
    _need(report, 4, "report")
    if query_start is not None:
        _need(query_start, R + 1, "query_start")
    _check(lib().pkv_check_tables(ctypes.byref(cache.desc), _dptr(block_tables, "block_tables", 4), stride,
                                  _dptr(context_lens, "context_lens", 4), R, int(max_context_len),
                                  _dptr(query_start, "query_start", 4),
                                  int(total_q), _dptr(report, "report", 4), _stream_ptr(stream)))


def prefill_workspace_size(cache: PagedCache, num_rows: int, total_q: int, max_q_per_row: int,
                           max_context_len: int) -> int:
    return int(lib().pkv_prefill_workspace_size(ctypes.byref(cache.desc), int(num_rows), int(total_q),
                                                int(max_q_per_row), int(max_context_len)))


def prefill_workspace_size_gqa(cache: PagedCache, num_q_heads: int, num_rows: int, total_q: int, max_q_per_row: int,
                               max_context_len: int) -> int:
    return int(lib().pkv_prefill_workspace_size_gqa(ctypes.byref(cache.desc), int(num_q_heads), int(num_rows),
                                                    int(total_q), int(max_q_per_row), int(max_context_len)))


def chunked_prefill_attention(cache: PagedCache, layer: int, out, q, query_start, block_tables, context_lens,
                              max_q_per_row: int, max_context_len: int, scale: float, workspace=None, stream=None):
    chunked_prefill_attention_gqa(cache, cache.num_heads, layer, out, q, query_start, block_tables, context_lens,
                                  max_q_per_row, max_context_len, scale, workspace, stream)


def chunked_prefill_attention_gqa(cache: PagedCache, num_q_heads: int, layer: int, out, q, query_start, block_tables,
                                  context_lens, max_q_per_row: int, max_context_len: int, scale: float,
                                  workspace=None, stream=None):
    R, stride = (int(x) for x in block_tables.shape)
    T = int(q.shape[0])
    _rows_need(T, num_q_heads, out=out, q=q)
    _need(query_start, R + 1, "query_start")
    _need(context_lens, R, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (int(layer), _dptr(out, "out", 2), _dptr(q, "q", 2), _dptr(query_start, "query_start", 4),
            _dptr(block_tables, "block_tables", 4), stride, _dptr(context_lens, "context_lens", 4), R, T,
            int(max_q_per_row), int(max_context_len), float(scale), _dptr(workspace, "workspace"), ws_bytes,
            _stream_ptr(stream))
    if int(num_q_heads) == cache.num_heads:  # one query head per KV head: the plain call
        _check(lib().pkv_chunked_prefill_attention(ctypes.byref(cache.desc), *args))
    else:
        _check(lib().pkv_chunked_prefill_attention_gqa(ctypes.byref(cache.desc), int(num_q_heads), *args))


# ------------------------------------------------------------------ whole blocks

def block_bytes(cache: PagedCache) -> int:
    """Bytes of one block with all its layers (one contiguous region of the pool)."""
    return int(lib().pkv_block_bytes(ctypes.byref(cache.desc)))


def copy_blocks(cache: PagedCache, src_ids, dst_ids, stream=None):
    """Copy-on-write: block src_ids[i] -> dst_ids[i], all layers (device int32 tensors)."""
    n = int(src_ids.numel())
    if int(dst_ids.numel()) != n:
        raise ValueError("src_ids and dst_ids must have the same length")
    _check(lib().pkv_copy_blocks(ctypes.byref(cache.desc), _dptr(src_ids, "src_ids", 4), _dptr(dst_ids, "dst_ids", 4),
                                 n, _stream_ptr(stream)))


def _host_buf(t, need: int, what: str):
    if t.is_cuda:
        raise ValueError(f"{what} must be host memory")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, needs {need}")
    return ctypes.c_void_p(t.data_ptr())


def swap_out(cache: PagedCache, ids, host_dst, stream=None):
    """Queue copies of blocks ids (host ints) into host_dst (a pinned host tensor),
    block i at byte offset i * block_bytes(cache)."""
    a = _i32(ids)
    buf = _host_buf(host_dst, len(a) * block_bytes(cache), "host_dst")
    _check(lib().pkv_swap_out(ctypes.byref(cache.desc), _iptr(a), len(a), buf, _stream_ptr(stream)))


def swap_in(cache: PagedCache, host_src, ids, stream=None):
    """Queue copies of host_src (a pinned host tensor), block i at byte offset
    i * block_bytes(cache), into blocks ids (host ints)."""
    a = _i32(ids)
    buf = _host_buf(host_src, len(a) * block_bytes(cache), "host_src")
    _check(lib().pkv_swap_in(ctypes.byref(cache.desc), buf, _iptr(a), len(a), _stream_ptr(stream)))


# ------------------------------------------------------------------ 8-bit cache

class PagedCache8:
    """Descriptor of a caller-owned 8-bit KV pool: codes [num_blocks, num_layers, 2,
    num_heads, 16, 128] of uint8 (FP8 E4M3) and scales [num_blocks, num_layers, 2,
    num_heads, 16] of float32, one per (token, head) row."""

    def __init__(self, codes, scales):
        if codes.dim() != 6 or codes.shape[2] != 2 or codes.shape[4] != BLOCK_SIZE or codes.shape[5] != HEAD_DIM:
            raise ValueError("codes must be [num_blocks, num_layers, 2, num_heads, 16, 128]")
        if tuple(scales.shape) != tuple(codes.shape[:5]):
            raise ValueError("scales must be [num_blocks, num_layers, 2, num_heads, 16]")
        _dptr(codes, "codes", 1)
        _dptr(scales, "scales", 4)
        self.codes, self.scales = codes, scales
        nb, nl, _, nh, bs, hd = (int(x) for x in codes.shape)
        self.desc = _lib.PkvCache8Desc(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                       nb, nl, nh, bs, hd)

    @property
    def num_heads(self) -> int:
        return int(self.desc.num_heads)


def append_fp8(cache: PagedCache8, layer: int, k_new, v_new, positions, request_of_token, block_tables,
               stream=None):
    T = int(positions.numel())
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(T, cache.num_heads, k_new=k_new, v_new=v_new)
    _need(request_of_token, T, "request_of_token")
    _check(lib().pkv_append_fp8(ctypes.byref(cache.desc), int(layer), _dptr(k_new, "k_new", 2),
                                _dptr(v_new, "v_new", 2), _dptr(positions, "positions", 4),
                                _dptr(request_of_token, "request_of_token", 4), T,
                                _dptr(block_tables, "block_tables", 4), R, stride, _stream_ptr(stream)))


def decode_workspace_size_fp8(cache: PagedCache8, num_rows: int, max_context_len: int) -> int:
    return int(lib().pkv_decode_workspace_size_fp8(ctypes.byref(cache.desc), int(num_rows), int(max_context_len)))


def decode_attention_append_fp8(cache: PagedCache8, layer: int, out, q, k_new, v_new, block_tables, context_lens,
                                max_context_len: int, scale: float, workspace=None, stream=None):
    """Quantize and append each row's new token at position context_lens[r] - 1, then decode (one fused launch)."""
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, cache.num_heads, out=out, q=q, k_new=k_new, v_new=v_new)
    _need(context_lens, R, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_attention_append_fp8(ctypes.byref(cache.desc), int(layer), _dptr(out, "out", 2),
                                                 _dptr(q, "q", 2), _dptr(k_new, "k_new", 2), _dptr(v_new, "v_new", 2),
                                                 _dptr(block_tables, "block_tables", 4), stride,
                                                 _dptr(context_lens, "context_lens", 4), R, int(max_context_len),
                                                 float(scale), _dptr(workspace, "workspace"), ws_bytes,
                                                 _stream_ptr(stream)))


def decode_attention_fp8(cache: PagedCache8, layer: int, out, q, block_tables, context_lens, max_context_len: int,
                         scale: float, workspace=None, stream=None):
    R, stride = (int(x) for x in block_tables.shape)
    _rows_need(R, cache.num_heads, out=out, q=q)
    _need(context_lens, R, "context_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_attention_fp8(ctypes.byref(cache.desc), int(layer), _dptr(out, "out", 2),
                                          _dptr(q, "q", 2), _dptr(block_tables, "block_tables", 4), stride,
                                          _dptr(context_lens, "context_lens", 4), R, int(max_context_len),
                                          float(scale), _dptr(workspace, "workspace"), ws_bytes, _stream_ptr(stream)))
