"""Continuous-batching decode loop over the paged KV cache.

Drives the hot path the way the serving loop on the pages does (LLM
inference batching, faangrind, scheduler steps 4-7; Inference
Infrastructure, seeitflow, "Why engines allocate in blocks"): every step
  * rows that have generated their answer leave and release their blocks,
  * waiting requests join; a prompt of at least `prefix_tokens` tokens shares
    the ref-counted prefix blocks and its remaining prompt tokens are appended
    into fresh private blocks ("fill"),
  * each running row grows its table when its next token starts a block,
    appends that token's K/V and runs decode attention over its context.
All bookkeeping goes through the library's block pool and all device work
through its kernels; this module only sequences the calls.

Token K/V values and queries are seeded draws (torch's device generator):
prompt tokens of request i from seed (seed, i), decode tokens and queries of
step s from seed (seed, s).  The `log` keeps what a checker needs to
rebuild any row's context independently.
"""
from __future__ import annotations

import dataclasses

import time

import numpy as np

from . import (BLOCK_SIZE, BlockPool, PagedCache, append, decode_attention_append, decode_attention_prefix,
               decode_workspace_size, decode_workspace_size_prefix)


def _seed(*parts: int) -> int:
    h = 1469598103934665603
    for p in parts:
        h = ((h ^ (int(p) & 0xFFFFFFFF)) * 1099511628211) & 0xFFFFFFFFFFFF
    return h


@dataclasses.dataclass
class Row:
    req: int
    prompt: int          # prompt tokens
    answer: int          # tokens to generate
    generated: int       # tokens generated so far
    shared: int          # leading tokens held in the shared prefix blocks
    slot: int            # row of the trace's table array this request occupies
    owner: "ContinuousBatchTrace"

    @property
    def length(self) -> int:  # tokens cached before this step's new token
        return self.prompt + self.generated

    @property
    def table(self) -> np.ndarray:  # int32 block ids (capacity = stride)
        return self.owner.tables[self.slot]

    @property
    def nblk(self) -> int:  # entries of `table` in use
        return int(self.owner.tlen[self.slot])


class ContinuousBatchTrace:
    STAGES = 4  # pinned upload buffers in the ring

    def __init__(self, torch, *, seed=3, num_blocks=36864, max_rows=64, prefix_tokens=2000,
                 prompt_range=(50, 8000), answer_range=(1, 1000), heads=32, stride=None, scale=None,
                 device="cuda", shared_decode=False):
        # shared_decode: decode through pkv_decode_attention_prefix, which reads
        # the shared prefix blocks once per step for every row holding them
        self.shared_decode = shared_decode
        self.torch = torch
        self.seed = seed
        self.H = heads
        self.max_rows = max_rows
        self.prefix_tokens = prefix_tokens - prefix_tokens % BLOCK_SIZE
        self.prompt_range = prompt_range
        self.answer_range = answer_range
        self.dev = torch.device(device)
        max_ctx = prompt_range[1] + answer_range[1]
        # the shared-prefix call needs the prefix's blocks to fit the table
        self.stride = stride or max(-(-max_ctx // BLOCK_SIZE), self.prefix_tokens // BLOCK_SIZE)
        self.scale = scale if scale is not None else 1.0 / np.sqrt(128.0)
        self.pool_d = torch.empty((num_blocks, 1, 2, heads, BLOCK_SIZE, 128), dtype=torch.float16, device=self.dev)
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(_seed(seed, 0xF111))
        self.pool_d.normal_(0.0, 1.0, generator=gen)
        self.cache = PagedCache(self.pool_d)
        rng = np.random.default_rng(seed)
        self.pool = BlockPool(num_blocks, rng.permutation(num_blocks).astype(np.int32))
        self.queue_rng = np.random.default_rng(_seed(seed, 0xA11))
        self.next_req = 0
        # the shared prefix: held once by the trace itself so it outlives its rows
        self.prefix_ids = self.pool.alloc(self.prefix_tokens // BLOCK_SIZE)
        # every row's block table lives in one slot of these arrays
        self.tables = np.zeros((max_rows, self.stride), dtype=np.int32)
        self.tlen = np.zeros(max_rows, dtype=np.int32)
        self.slot_row: list[Row | None] = [None] * max_rows
        self.step_no = 0
        self.max_ctx = max_ctx
        if shared_decode:
            ws = decode_workspace_size_prefix(self.cache, max_rows, max_ctx, self.prefix_tokens // BLOCK_SIZE)
        else:
            ws = decode_workspace_size(self.cache, max_rows, max_ctx)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.dev)
        # step metadata: a ring of pinned host buffers, each step's tables,
        # lengths, positions and marks copied asynchronously in one transfer
        # into one device array that every step reuses
        n_meta = max_rows * self.stride + 3 * max_rows
        self._stage = [torch.empty(n_meta, dtype=torch.int32, pin_memory=True) for _ in range(self.STAGES)]
        self._stage_done = [None] * self.STAGES
        self.meta_d = torch.empty(n_meta, dtype=torch.int32, device=self.dev)
        self.rot_d = torch.arange(max_rows, dtype=torch.int32, device=self.dev)
        self.log = {"prefix_ids": self.prefix_ids.copy(), "joins": [], "steps": []}

    @property
    def rows(self) -> list[Row]:
        """Running rows in step order (by slot)."""
        return [r for r in self.slot_row if r is not None]

    # ---------------------------------------------------------------- requests

    def _draw_request(self):
        p = int(self.queue_rng.integers(self.prompt_range[0], self.prompt_range[1] + 1))
        a = int(self.queue_rng.integers(self.answer_range[0], self.answer_range[1] + 1))
        req = self.next_req
        self.next_req += 1
        return req, p, a

    def prompt_kv(self, req: int, first: int, last: int):
        """Seeded K/V of prompt tokens first..last-1 of request `req`, [n, H, 128] each."""
        torch = self.torch
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(_seed(self.seed, 0xB0B, req))
        n_all = last  # draw the whole prompt so any sub-range is reproducible
        kv = torch.randn((2, n_all, self.H, 128), generator=gen, device=self.dev, dtype=torch.float16)
        return kv[0, first:last].contiguous(), kv[1, first:last].contiguous()

    def step_draws(self, step: int, n: int):
        """Seeded new-token K/V and queries of a step, [n, H, 128] each."""
        torch = self.torch
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(_seed(self.seed, 0x57E9, step))
        x = torch.randn((3, max(n, 1), self.H, 128), generator=gen, device=self.dev, dtype=torch.float16)
        return x[0, :n].contiguous(), x[1, :n].contiguous(), x[2, :n].contiguous()

    def _join(self, slot, req, prompt, answer):
        torch = self.torch
        table = self.tables[slot]
        table[:] = 0
        shared = self.prefix_tokens if prompt >= self.prefix_tokens else 0
        nblk = 0
        if shared:
            nshared = shared // BLOCK_SIZE
            self.pool.ref(self.prefix_ids)
            table[:nshared] = self.prefix_ids
            nblk = nshared
        self.tlen[slot] = self.pool.grow(table, nblk, prompt)
        row = Row(req, prompt, answer, 0, shared, slot, self)
        # fill: the private prompt tokens' K/V go into the fresh blocks
        if prompt > shared:
            k, v = self.prompt_kv(req, shared, prompt)
            pos = torch.arange(shared, prompt, dtype=torch.int32, device=self.dev)
            rot = torch.zeros(prompt - shared, dtype=torch.int32, device=self.dev)
            tab = torch.from_numpy(table[None, :].copy()).to(self.dev)
            append(self.cache, 0, k, v, pos, rot, tab)
        self.log["joins"].append((req, prompt, answer, shared, self.step_no))
        return row

    def _leave(self, row: Row):
        self.pool.free(self.tables[row.slot, :row.nblk])
        self.tlen[row.slot] = 0
        self.slot_row[row.slot] = None

    # ---------------------------------------------------------------- one step

    def step(self, events=None, before_decode=None):
        """Leave, join, grow, append one token per row, decode.  Returns the
        step's row snapshot (for checkers).  With events=(start, filled,
        launch, end) it records them around the fill of joining rows and
        around the decode part's launches.  The host's preparation of the step
        (one batched table growth through the block pool, and the staging and
        asynchronous upload of tables, lengths and marks through pinned
        memory) is timed on the host and returned as snap["host_ms"]; the
        step's synthetic inputs are drawn before it and not counted, and the
        wait for a free staging buffer (the host running ahead of the GPU) is
        returned apart as snap["stage_wait_ms"].
        before_decode, if given, is called just before the decode part is
        queued (e.g. to scrub the caches)."""
        torch = self.torch
        for r in self.rows:
            if r.generated >= r.answer:
                self._leave(r)
        if events:
            events[0].record()
        for slot in range(self.max_rows):
            if self.slot_row[slot] is None:
                self.slot_row[slot] = self._join(slot, *self._draw_request())
        if events:
            events[1].record()
        rows = self.rows
        R = len(rows)
        k, v, q = self.step_draws(self.step_no, R)
        out = torch.empty((R, self.H, 128), dtype=torch.float16, device=self.dev)

        t_host = time.perf_counter()
        slots = np.array([r.slot for r in rows], dtype=np.int64)
        lens = np.array([r.length + 1 for r in rows], dtype=np.int32)
        need = np.zeros(self.max_rows, dtype=np.int32)
        need[slots] = lens  # the new token sits at position r.length
        grown = self.pool.grow_rows(self.tables, self.tlen, need)
        if grown < self.max_rows:
            raise RuntimeError("block pool exhausted: the trace's pool is sized so that every row always fits")
        st = self.step_no % self.STAGES
        wait_ms = 0.0
        if self._stage_done[st] is not None:
            # its previous upload has landed; a host that runs ahead of the
            # GPU waits here, which is backpressure, not preparation
            t_wait = time.perf_counter()
            self._stage_done[st].synchronize()
            wait_ms = (time.perf_counter() - t_wait) * 1e3
        buf = self._stage[st]
        a = buf.numpy()
        n_tab = R * self.stride
        a[:n_tab] = self.tables[slots].reshape(-1)
        a[n_tab:n_tab + R] = lens
        a[n_tab + R:n_tab + 2 * R] = lens - 1
        a[n_tab + 2 * R:n_tab + 3 * R] = [1 if r.shared else 0 for r in rows]
        n = n_tab + 3 * R
        self.meta_d[:n].copy_(buf[:n], non_blocking=True)
        tab_d = self.meta_d[:n_tab].view(R, self.stride)
        lens_d = self.meta_d[n_tab:n_tab + R]
        pos_d = self.meta_d[n_tab + R:n_tab + 2 * R]
        marks_d = self.meta_d[n_tab + 2 * R:n]
        rot_d = self.rot_d[:R]
        ev = torch.cuda.Event()
        ev.record()
        self._stage_done[st] = ev
        host_ms = (time.perf_counter() - t_host) * 1e3 - wait_ms
        if before_decode is not None:
            before_decode()
        if events:
            events[2].record()
        if self.shared_decode:
            append(self.cache, 0, k, v, pos_d, rot_d, tab_d)
            decode_attention_prefix(self.cache, 0, out, q, tab_d, lens_d, self.max_ctx, self.scale, marks_d,
                                    self.prefix_tokens // BLOCK_SIZE, self.ws)
        else:
            # each row's new token is appended by the decode launch itself
            decode_attention_append(self.cache, 0, out, q, k, v, tab_d, lens_d, self.max_ctx, self.scale, self.ws)
        if events:
            events[3].record()
        tables = self.tables[slots].copy()
        snap = {"step": self.step_no, "reqs": [r.req for r in rows], "lens": lens.copy(),
                "gen_index": [r.generated for r in rows], "tables": tables, "out": out, "host_ms": host_ms,
                "stage_wait_ms": wait_ms}
        self.log["steps"].append({"step": self.step_no, "reqs": snap["reqs"], "lens": lens.copy(),
                                  "new_pos": (lens - 1).copy()})
        for r in rows:
            r.generated += 1
        self.step_no += 1
        return snap

    def drain(self):
        for r in self.rows:
            self._leave(r)
        self.pool.free(self.prefix_ids)
