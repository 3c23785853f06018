"""Seeded synthetic batches shaped like the serving workloads the pages describe.

Model shape (LLM inference batching, faangrind: "Model" and "KV cache"): a
7B model with 32 layers, 32 heads of dimension 128, FP16 keys and values, and a
pool of 16-token blocks laid out per block as [layers, 2, heads, 16, 128].
Prompt and answer length ranges come from the same page's problem statement
(prompts 50 to 8,000 tokens, answers 1 to 1,000 tokens).

What this module draws, and nothing more:
  * per-row context lengths and query counts,
  * a seeded permutation used as the initial free list, and block tables cut
    from its top in the order a last-in-first-out free list hands ids out,
  * N(0,1) FP16 values for queries, new keys/values and the pool contents,
    with NaN written into every slot that holds no live token (unowned
    blocks, slots at or past a row's first new position) so that a stray
    read shows up in the outputs.

Everything is returned as NumPy arrays (FP16 data as uint16 bit patterns) or,
for pools too large for host memory, filled on the device by
`fill_normal_fp16_device`.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEADS = 32
HEAD_DIM = 128
BLOCK = 16
SCALE = 1.0 / math.sqrt(HEAD_DIM)
F16_QNAN = np.uint16(0x7E00)

__all__ = [
    "HEADS", "HEAD_DIM", "BLOCK", "SCALE", "F16_QNAN", "Batch", "build_batch",
    "c1_tiny", "c2_average_mix", "c3_long_context", "c5_mixed", "c2_lengths",
    "trace_requests", "fill_normal_fp16_device", "normal_f16_bits",
]


def normal_f16_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) drawn in float32, rounded to FP16, returned as uint16 bits."""
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16).view(np.uint16)


@dataclass
class Batch:
    """One step's worth of inputs for a single layer shape.

    context_lens[r]   keys visible to row r's last query, counting the new tokens
    q_counts[r]       queries (and new tokens) of row r; 1 marks a decode row
    query_start       exclusive prefix sum of q_counts, [R+1]
    positions, request_of_token   [T]: where each new token goes
    q, k_new, v_new   [NLq, T, H, D] uint16 (FP16 bits), one slice per layer
    block_tables      [R, stride] int32; entries past a row's last block hold
                      an unowned (poisoned) block id when one exists
    free_list         the seeded permutation the tables were cut from
    pool              [NB, NL, 2, H, 16, D] uint16 before the append, or None
    """

    name: str
    seed: int
    num_blocks: int
    num_layers: int
    num_heads: int
    context_lens: np.ndarray
    q_counts: np.ndarray
    query_start: np.ndarray
    positions: np.ndarray
    request_of_token: np.ndarray
    block_tables: np.ndarray
    free_list: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    pool: np.ndarray | None = None
    free_after: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.query_start[-1])

    @property
    def bt_stride(self) -> int:
        return int(self.block_tables.shape[1])


def build_batch(name: str, seed: int, lens, q_counts, *, num_blocks: int, num_layers: int = 1,
                num_heads: int = HEADS, stride: int | None = None, layers_with_q: int | None = None,
                with_pool: bool = True, poison: bool = True, shared_prefix_blocks: int = 0,
                shared_rows=None) -> Batch:
    """Draw a batch.

    lens[r] is the context length after the new tokens; q_counts[r] new tokens
    (and queries) per row.  Rows take ceil(lens[r] / 16) block ids from the top
    of a seeded permutation, row 0 first.  With shared_prefix_blocks = P, rows
    listed in shared_rows point their first P table entries at the first P ids
    row 0 took (a ref-counted prefix); those rows take only their remaining
    blocks from the list.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    q_counts = np.asarray(q_counts, dtype=np.int64)
    R = lens.shape[0]
    if np.any(lens < 1) or np.any(q_counts < 1) or np.any(q_counts > lens):
        raise ValueError("need 1 <= q_counts[r] <= lens[r]")
    nblk = (lens + BLOCK - 1) // BLOCK
    if stride is None:
        stride = int(nblk.max())
    if int(nblk.max()) > stride:
        raise ValueError("stride too small for the longest row")
    shared_rows = set() if shared_rows is None else set(int(r) for r in shared_rows)
    perm = rng.permutation(num_blocks).astype(np.int32)
    stack = list(perm)
    tables = np.zeros((R, stride), dtype=np.int32)
    owned = np.zeros(num_blocks, dtype=bool)
    prefix_ids = None
    for r in range(R):
        start = 0
        if r in shared_rows and prefix_ids is not None:
            take = min(shared_prefix_blocks, int(nblk[r]))
            tables[r, :take] = prefix_ids[:take]
            start = take
        for j in range(start, int(nblk[r])):
            if not stack:
                raise ValueError("pool too small for the batch")
            tables[r, j] = stack.pop()
            owned[tables[r, j]] = True
        if r == 0 and shared_prefix_blocks:
            prefix_ids = tables[0, :shared_prefix_blocks].copy()
    free_after = np.array(stack, dtype=np.int32)
    filler = int(free_after[0]) if free_after.size else int(tables[0, 0])
    for r in range(R):
        tables[r, int(nblk[r]):] = filler

    query_start = np.zeros(R + 1, dtype=np.int32)
    query_start[1:] = np.cumsum(q_counts)
    T = int(query_start[-1])
    positions = np.concatenate([np.arange(lens[r] - q_counts[r], lens[r]) for r in range(R)]).astype(np.int32)
    request_of_token = np.repeat(np.arange(R), q_counts).astype(np.int32)

    nlq = num_layers if layers_with_q is None else layers_with_q
    H, D = num_heads, HEAD_DIM
    q = normal_f16_bits(rng, (nlq, T, H, D))
    k_new = normal_f16_bits(rng, (nlq, T, H, D))
    v_new = normal_f16_bits(rng, (nlq, T, H, D))

    pool = None
    if with_pool:
        shape = (num_blocks, num_layers, 2, H, BLOCK, D)
        pool = normal_f16_bits(rng, shape)
        if poison:
            pool[~owned] = F16_QNAN
            # slots at or after a row's first new position hold no live token yet
            for r in range(R):
                first_new = int(lens[r] - q_counts[r])
                for j in range(first_new // BLOCK, int(nblk[r])):
                    b = int(tables[r, j])
                    s0 = max(first_new - j * BLOCK, 0)
                    pool[b, :, :, :, s0:, :] = F16_QNAN
    return Batch(name=name, seed=seed, num_blocks=num_blocks, num_layers=num_layers, num_heads=num_heads,
                 context_lens=lens.astype(np.int32), q_counts=q_counts.astype(np.int32),
                 query_start=query_start, positions=positions, request_of_token=request_of_token,
                 block_tables=tables, free_list=perm, q=q, k_new=k_new, v_new=v_new, pool=pool,
                 free_after=free_after)


def c1_tiny(seed: int = 0) -> Batch:
    """Tiny decode: one layer, 64-block pool, 4 rows with contexts 17, 40, 100, 256."""
    return build_batch("tiny-decode-4x{17,40,100,256}", seed, [17, 40, 100, 256], [1, 1, 1, 1],
                       num_blocks=64, num_layers=1, stride=16)


def c2_lengths(rng: np.random.Generator, rows: int) -> np.ndarray:
    """Average-mix contexts: lognormal prompt (pre-clip mean 1,250, sigma 1) clipped
    to [50, 8000], plus U{1..300} generated tokens."""
    sigma = 1.0
    mu = math.log(1250.0) - sigma * sigma / 2.0
    prompt = np.clip(np.rint(rng.lognormal(mu, sigma, rows)), 50, 8000).astype(np.int64)
    generated = rng.integers(1, 301, rows)
    return prompt + generated


def c2_average_mix(seed: int = 1, *, rows: int = 32, with_pool: bool = False, num_layers: int = 32,
                   num_blocks: int = 7152) -> Batch:
    """Average-mix decode step: 32 rows over a 7,152-block, 32-layer pool."""
    rng = np.random.default_rng(seed + 1000)
    lens = c2_lengths(rng, rows)
    return build_batch(f"average-mix-decode-{rows}rows-{num_layers}layers", seed, lens, np.ones(rows),
                       num_blocks=num_blocks, num_layers=num_layers, stride=520, with_pool=with_pool,
                       poison=False)


def c3_long_context(seed: int = 2, *, rows: int = 13, with_pool: bool = False, num_layers: int = 32,
                    num_blocks: int = 7152) -> Batch:
    """Long-context decode: 13 rows of 8,192 tokens (512 blocks each)."""
    return build_batch(f"long-context-decode-{rows}x8192-{num_layers}layers", seed, [8192] * rows,
                       np.ones(rows), num_blocks=num_blocks, num_layers=num_layers, stride=512,
                       with_pool=with_pool, poison=False)


def c5_mixed(seed: int = 4, *, chunk: int = 512, prompt: int = 8000, decode_rows: int = 31,
             with_pool: bool = False, num_blocks: int = 7152, poison: bool = False) -> Batch:
    """Chunked prefill mixed with decode: one row whose last `chunk` prompt tokens
    (positions prompt-chunk .. prompt-1) are the chunk, then `decode_rows` decode
    rows drawn like the average mix.  One layer."""
    rng = np.random.default_rng(seed + 1000)
    lens = np.concatenate([[prompt], c2_lengths(rng, decode_rows)])
    qc = np.concatenate([[chunk], np.ones(decode_rows, dtype=np.int64)])
    return build_batch(f"mixed-prefill{chunk}@{prompt - chunk}+{decode_rows}decode", seed, lens, qc,
                       num_blocks=num_blocks, num_layers=1, stride=520, with_pool=with_pool, poison=poison)


def trace_requests(seed: int, count: int):
    """Request queue for the continuous-batching trace: prompt U{50..8000},
    output U{1..1000}."""
    rng = np.random.default_rng(seed)
    prompts = rng.integers(50, 8001, count)
    outputs = rng.integers(1, 1001, count)
    return prompts.astype(np.int64), outputs.astype(np.int64)


def fill_normal_fp16_device(tensor, seed: int, chunk_elems: int = 1 << 28) -> None:
    """Fill a (large) FP16 device tensor with seeded N(0,1) values in chunks."""
    import torch

    gen = torch.Generator(device=tensor.device)
    gen.manual_seed(int(seed))
    flat = tensor.view(torch.float16).view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        flat[s:s + chunk_elems].normal_(0.0, 1.0, generator=gen)
