"""Paged KV cache oracle: append, gather, attention.  float64 NumPy on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pool layout (LLM inference batching, faangrind, data model "KV pool"): every
16-token block holds [layers, 2, heads, 16 tokens, head_dim] FP16 values, key
first (index 0) and value second (index 1).  The pool array handled here is
[num_blocks, layers, 2, heads, 16, head_dim] of uint16 bit patterns, so that
append compares bit for bit.

Arrays indexed by block id ("pool_layer") may be any object with
`pool_layer[b] -> [2, heads, 16, head_dim]`: a NumPy view `pool[:, layer]`, or a
dict holding only the blocks that were read back.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


def locate(table_row, position: int, block_size: int = BLOCK_SIZE):
    """Physical (block id, slot) of logical token `position` of a row.

    A row takes a new block every 16 tokens (LLM inference batching, faangrind,
    scheduler step 7), so token j lives in logical block j // 16 at slot
    j % 16, and the row's block table maps the logical block to a physical one
    (Build a continuous batching server, scalablesystem.dev, "PagedAttention
    Block Table Lookup").
    """
    return int(table_row[position // block_size]), position % block_size


def append(pool: np.ndarray, layer: int, k_new, v_new, positions, request_of_token, block_tables) -> np.ndarray:
    """Return a copy of `pool` with each new token's key and value written.

    The decode step appends the new token's keys and values into its row's
    current block (LLM inference batching, faangrind, scheduler step 7; The
    inference engine, wpnews, "Paging turns variable sequences into block
    tables": the next token fills the current block).  Token t of the step
    belongs to row request_of_token[t] at position positions[t] (the flat,
    request-tagged token list of the same page's step tensors).  k_new and
    v_new are [T, heads, head_dim] FP16 (or their uint16 bits).  Tokens are
    written in order t = 0, 1, ...
    """
    out = np.array(pool, copy=True)
    kb = np.ascontiguousarray(k_new).view(np.uint16)
    vb = np.ascontiguousarray(v_new).view(np.uint16)
    for t in range(len(positions)):
        r = int(request_of_token[t])
        b, s = locate(block_tables[r], int(positions[t]))
        out[b, layer, 0, :, s, :] = kb[t]
        out[b, layer, 1, :, s, :] = vb[t]
    return out


def gather_kv(pool_layer, table_row, seq_len: int, block_size: int = BLOCK_SIZE):
    """Contiguous K and V of one row as float64 [heads, seq_len, head_dim].

    The gather walks the row's full blocks, then takes the first
    seq_len % block_size tokens of the next one, and concatenates them in
    logical order (Build a continuous batching server, scalablesystem.dev,
    "PagedAttention Block Table Lookup").  That page's pool is token-major;
    here each block slab is [2, heads, 16, head_dim] as the faangrind data
    model gives it, so tokens are concatenated along axis 1.
    """
    num_full, remainder = divmod(int(seq_len), block_size)
    keys, values = [], []
    for i in range(num_full):
        slab = np.asarray(pool_layer[int(table_row[i])])
        keys.append(slab[0])
        values.append(slab[1])
    if remainder:
        slab = np.asarray(pool_layer[int(table_row[num_full])])
        keys.append(slab[0][:, :remainder])
        values.append(slab[1][:, :remainder])
    K = np.concatenate(keys, axis=1)
    V = np.concatenate(values, axis=1)
    return _f64(K), _f64(V)


def _f64(bits) -> np.ndarray:
    a = np.ascontiguousarray(bits)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    return a.astype(np.float64)


def attention(q, K, V, query_positions, scale: float) -> np.ndarray:
    """Scaled dot-product attention with a causal rule, float64.

    q is [n, heads, head_dim]; K, V are [heads, L, head_dim].  Query i sits at
    position query_positions[i] and sees keys 0 .. query_positions[i]
    inclusive: a decode token's attention reads every cached position
    including its own freshly appended one (Inference Infrastructure,
    seeitflow, "Three iterations with the state written out"), and prefill
    respects the causal mask (The inference engine, wpnews, "Prefill and
    decode ask the accelerator for different work").  Scores are
    (q . k) * scale; the softmax subtracts the row maximum before
    exponentiating, which leaves its value unchanged.
    """
    q = _f64(q)
    n, H, D = q.shape
    L = K.shape[1]
    pos = np.asarray(query_positions, dtype=np.int64).reshape(n)
    if np.any(pos < 0) or np.any(pos >= L):
        raise ValueError("query position outside the context")
    hidden = np.arange(L)[None, :] > pos[:, None]
    out = np.empty((n, H, D), dtype=np.float64)
    for h in range(H):
        S = (q[:, h, :] @ K[h].T) * scale
        S[hidden] = -np.inf
        m = S.max(axis=1, keepdims=True)
        W = np.exp(S - m)
        out[:, h, :] = (W @ V[h]) / W.sum(axis=1, keepdims=True)
    return out


def group_kv(K, V, group: int):
    """Keys and values as seen by each query head under grouped-query
    attention: one K/V head is shared by a group of `group` query heads
    (Inference Infrastructure, seeitflow: MHA keeps one K/V pair per query
    head, GQA shares one K/V head among a group of query heads).  The pages do
    not say which query heads form a group; consecutive heads do here, so query
    head h reads KV head h // group.  group = 1 is plain multi-head attention."""
    if group == 1:
        return K, V
    return np.repeat(K, group, axis=0), np.repeat(V, group, axis=0)


def decode(pool_layer, q, block_tables, context_lens, scale: float, rows=None, group: int = 1) -> np.ndarray:
    """One query per row at position context_lens[r] - 1, over that row's
    gathered context.  q is [R, heads * group, head_dim]; returns that shape
    (or only the listed rows, in the order given)."""
    rows = range(len(context_lens)) if rows is None else rows
    outs = []
    for r in rows:
        L = int(context_lens[r])
        K, V = group_kv(*gather_kv(pool_layer, block_tables[r], L), group)
        outs.append(attention(np.asarray(q)[r:r + 1], K, V, [L - 1], scale)[0])
    return np.stack(outs)


def chunked_prefill(pool_layer, q, query_start, block_tables, context_lens, scale: float, rows=None,
                    group: int = 1) -> np.ndarray:
    """Row r owns queries query_start[r] .. query_start[r+1]-1, which are the last
    n_r positions of its context, L_r - n_r .. L_r - 1.  A row with n_r = 1 is
    a decode row.  Prefill chunks and decode rows share one step as a flat list
    of tokens tagged with their request (LLM inference batching, faangrind,
    "Prefill and decode share each step").  q has heads * group query heads
    (see group_kv).  Returns [T, heads * group, head_dim], or for `rows` the
    concatenation of those rows' query outputs."""
    qs = np.asarray(query_start)
    rows = range(len(context_lens)) if rows is None else rows
    outs = []
    for r in rows:
        L = int(context_lens[r])
        a, b = int(qs[r]), int(qs[r + 1])
        n = b - a
        K, V = group_kv(*gather_kv(pool_layer, block_tables[r], L), group)
        outs.append(attention(np.asarray(q)[a:b], K, V, np.arange(L - n, L), scale))
    return np.concatenate(outs, axis=0)
