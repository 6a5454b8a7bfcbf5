"""Host-side block bookkeeping used to build synthetic paged-KV inputs.

This is the allocator and reference counting that a serving engine keeps on
the host (PagedAttention - Efficient Memory Management for LLM Serving with
vLLM, irregular6612.github.io, "Method" and "Core components": free list of
physical blocks, per-block reference counts, per-sequence block tables,
copy-on-write when a shared block is about to be written).  Here it only
produces the inputs of the GPU calls: block tables, slot mappings and
(src, dst) copy pairs.  It performs none of the attention arithmetic.

Conventions (stated in the design notes as readings of the pages):
* A sequence of n tokens holds ceil(n / B) blocks; token t lives in logical
  block t // B at offset t % B.
* slot = physical_block * B + offset.
* The free list is a seeded random permutation of the pool, so physical
  placement is arbitrary; blocks are taken from its front in request order.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, order: np.ndarray):
        if sorted(order.tolist()) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(int(b) for b in order)
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    def allocate(self) -> int:
        if not self.free:
            raise PoolExhausted("no free KV block left in the pool")
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def share(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] += 1

    def release(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    @property
    def used(self) -> int:
        return int((self.ref > 0).sum())


@dataclass
class SeqBlocks:
    """Block table and token count of one sequence."""

    table: List[int] = field(default_factory=list)
    length: int = 0


def append_tokens(pool: BlockPool, seq: SeqBlocks, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
    """Reserve slots for ``n`` new tokens of ``seq``.

    A new block is taken only when the current last block is full.  If the
    block about to receive a write is shared (reference count above one), the
    writer first takes a private copy: a fresh block is allocated, the pair
    (shared, fresh) is recorded for a block copy, and the table entry is
    replaced.  Returns the slots of the new tokens and the copy pairs.
    """
    B = pool.block_size
    slots: List[int] = []
    pairs: List[Tuple[int, int]] = []
    for _ in range(n):
        pos = seq.length
        j, off = divmod(pos, B)
        if j == len(seq.table):
            seq.table.append(pool.allocate())
        else:
            b = seq.table[j]
            if pool.ref[b] > 1:
                nb = pool.allocate()
                pairs.append((b, nb))
                pool.release(b)
                seq.table[j] = nb
        slots.append(seq.table[j] * B + off)
        seq.length += 1
    return slots, pairs


def fork(pool: BlockPool, parent: SeqBlocks, n: int) -> List[SeqBlocks]:
    """Replace ``parent`` by ``n`` children that share all of its blocks."""
    kids = []
    for _ in range(n):
        for b in parent.table:
            pool.share(b)
        kids.append(SeqBlocks(list(parent.table), parent.length))
    for b in parent.table:
        pool.release(b)
    parent.table = []
    parent.length = 0
    return kids


def cow_last_block(pool: BlockPool, seq: SeqBlocks) -> List[Tuple[int, int]]:
    """Give ``seq`` a private copy of its partially filled last block if shared."""
    if not seq.table or seq.length % pool.block_size == 0:
        return []
    j = len(seq.table) - 1
    b = seq.table[j]
    if pool.ref[b] <= 1:
        return []
    nb = pool.allocate()
    pool.release(b)
    seq.table[j] = nb
    return [(b, nb)]


def tables_array(seqs: List[SeqBlocks], width: int | None = None, pad: int = -1) -> np.ndarray:
    """Pack block tables into an int32 [S, width] array padded with ``pad``."""
    w = max(1, max(len(s.table) for s in seqs)) if width is None else width
    out = np.full((len(seqs), w), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        out[i, : len(s.table)] = s.table
    return out
