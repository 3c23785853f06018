"""Whole-block copies of the paged KV pool: copy-on-write and swap.  NumPy on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A block with all its layers is the sub-array pool[b] of the
[num_blocks, layers, 2, heads, 16, head_dim] pool (LLM inference batching,
faangrind, data model "KV pool": one block holds every layer's keys and
values for 16 tokens).  Arrays hold uint16 bit patterns, so copies compare
bit for bit.
"""
from __future__ import annotations

import numpy as np


def copy_blocks(pool: np.ndarray, src_ids, dst_ids) -> np.ndarray:
    """Return a copy of `pool` in which block dst_ids[i] holds the bits of block
    src_ids[i], every layer, keys and values.

    Requests sharing prefix blocks hold them immutable; a branch that diverges
    inside a shared block first takes a private copy of it (The inference
    engine, wpnews.pro, "Weights, activations, and KV state occupy different
    ledgers": copy-on-write restores separate ownership when a branch
    diverges).  Pairs with an id outside the pool are skipped.  Destinations
    are distinct and are not sources of the same call, so every copy reads the
    pool as it was before the call.
    """
    nb = pool.shape[0]
    out = pool.copy()
    for s, d in zip(np.asarray(src_ids).tolist(), np.asarray(dst_ids).tolist()):
        if 0 <= s < nb and 0 <= d < nb:
            out[d] = pool[s]
    return out


def swap_out(pool: np.ndarray, ids) -> np.ndarray:
    """Host image of blocks `ids`: entry i is block ids[i], all layers.

    Under memory pressure a scheduler may move a sequence's blocks to host
    memory and restore them later rather than recompute its prefill (Build a
    continuous batching server, scalablesystem.dev, "Preemption and Eviction:
    Recompute vs Swap").
    """
    return np.stack([pool[int(b)] for b in ids]) if len(ids) else pool[:0].copy()


def swap_in(pool: np.ndarray, host: np.ndarray, ids) -> np.ndarray:
    """Return a copy of `pool` with host entry i written to block ids[i]
    (restoring swapped-out blocks, possibly at other physical ids)."""
    out = pool.copy()
    for i, b in enumerate(ids):
        out[int(b)] = host[i]
    return out
