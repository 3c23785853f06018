"""Python model of the KV block pool.  TEST INFRASTRUCTURE ONLY.

Follows the block managers the pages print and describe:
  * a free list that hands out ids with pop() from its end and takes them back
    by appending (Build a continuous batching server, scalablesystem.dev,
    "The KV Cache Block Manager (PagedAttention)"; Serving LLMs, sreshtalluri,
    "Paged KV memory" BlockPool);
  * blocks_needed(n) = ceil(n / 16);
  * allocation is all-or-nothing: when the free list is short nothing changes
    and the caller must preempt someone (Serving LLMs, BlockPool.grow);
  * a reference count per block, above 1 while samples or prefixes share it;
    a block returns to the free list only when its count reaches zero
    (LLM inference batching, faangrind, data model and failure list).
"""
from __future__ import annotations

from collections import Counter

BLOCK_SIZE = 16


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class DoubleFree(PoolError):
    pass


class BadBlock(PoolError):
    pass


def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """ceil(num_tokens / block_size)."""
    return -(-int(num_tokens) // block_size)


class BlockPool:
    def __init__(self, num_blocks: int, free_list=None):
        """Pool of num_blocks ids.  Without free_list the free list is
        0 .. num_blocks-1 (the next allocation takes num_blocks-1).  With one,
        it must list distinct ids; ids not on it start held once (count 1)."""
        self.num_blocks = int(num_blocks)
        if free_list is None:
            free_list = range(self.num_blocks)
        self.free = [int(b) for b in free_list]
        if len(set(self.free)) != len(self.free) or any(not 0 <= b < self.num_blocks for b in self.free):
            raise BadBlock("free list must hold distinct ids in range")
        self.ref = [1] * self.num_blocks
        for b in self.free:
            self.ref[b] = 0

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, n: int) -> list[int]:
        if n < 0:
            raise PoolError("negative count")
        if n > len(self.free):
            raise OutOfBlocks(f"need {n}, have {len(self.free)}")
        ids = [self.free.pop() for _ in range(n)]
        for b in ids:
            self.ref[b] = 1
        return ids

    def share(self, ids) -> None:
        ids = [int(b) for b in ids]
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise BadBlock(str(b))
            if self.ref[b] == 0:
                raise DoubleFree(f"block {b} is free")
        for b in ids:
            self.ref[b] += 1

    def release(self, ids) -> None:
        ids = [int(b) for b in ids]
        for b in ids:
            if not 0 <= b < self.num_blocks:
                raise BadBlock(str(b))
        for b, c in Counter(ids).items():
            if self.ref[b] < c:
                raise DoubleFree(f"block {b} released {c} times with count {self.ref[b]}")
        for b in ids:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def grow(self, table: list[int], num_tokens: int) -> bool:
        """Make `table` cover num_tokens; False (and no change) when short."""
        need = blocks_needed(num_tokens) - len(table)
        if need <= 0:
            return True
        if need > len(self.free):
            return False
        table.extend(self.alloc(need))
        return True
