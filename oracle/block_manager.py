"""Reference model of the KV-cache block manager.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's
CPU-baseline leg may import or run this module; the library's own block
manager (C++) shares no code with it.  Plain Python, one operation at a
time, written from the pages:

* PagedAttention digest (irregular6612.github.io), "Method" (core
  components: the block manager keeps the free list of physical blocks,
  per-block reference counts and the copy-on-write trigger; blocks are
  allocated only as tokens arrive) and its flowchart (two sequences share a
  physical block; a write to the shared block copies it first);
* the page on vLLM PagedAttention and continuous batching
  (tech.blogsailing.com), section 2 (forked samples share the prompt's
  blocks by raising the reference count; blocks are duplicated only at the
  branch point) and section 4 (blocks needed = ceil(tokens / B); a finished
  sequence's blocks return to the free pool);
* the KV-cache page (allinfo.ai.kr), key insights: with prefix caching,
  requests that share a prefix (a system prompt) point at the same physical
  blocks and skip that part of the prefill;
* the digest's scheduling and glossary: a preempted request's blocks can be
  swapped to CPU RAM and back.

Readings taken where the pages leave the policy open (the C++ manager
implements the same ones, so the two agree block id for block id):
* the free list is first-in first-out, starting from a given order;
* appending n tokens first checks that the blocks it needs (new blocks plus
  one copy when the partly filled last block is shared) are available, and
  changes nothing when they are not;
* a block is identified for prefix caching once it is full, by its tokens
  and the identity of the sequence's block before it, i.e. by the whole
  token prefix up to its end (whether or not that earlier block is the
  cached one); the first full block with a given identity is the cached
  one;
* a new sequence reuses the cached blocks of its prompt's longest cached
  prefix of whole blocks, but always leaves at least one prompt token to be
  computed;
* a cached block whose reference count drops to zero stays cached and
  becomes evictable; allocation takes plain free blocks first, then evicts
  the least recently released cached block;
* freeing a sequence releases its blocks from the first to the last;
* swapping a sequence out copies every block to a host pool (pairs device
  block -> host block, in table order) and releases the device blocks;
  swapping in is the reverse, onto freshly allocated device blocks.
"""
from __future__ import annotations

from collections import OrderedDict, deque
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None,
                 prefix_cache: bool = False):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.B = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.tokens: Dict[int, List[int]] = {}
        self.keys: Dict[int, List[tuple]] = {}  # per sequence: identity of each full block
        self.prefix_cache = prefix_cache
        self.cache: Dict[tuple, int] = {}      # prefix identity -> cached block
        self.key_of: Dict[int, tuple] = {}     # cached block -> its prefix identity
        self.evictable: "OrderedDict[int, None]" = OrderedDict()  # released cached blocks, LRU first

    # ----------------------------------------------------------- blocks
    def num_free(self) -> int:
        return len(self.free) + len(self.evictable)

    def _allocate(self) -> int:
        if self.free:
            b = self.free.popleft()
        elif self.evictable:
            b, _ = self.evictable.popitem(last=False)
            del self.cache[self.key_of.pop(b)]
        else:
            raise OutOfBlocks("no free block")
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        assert self.ref[b] > 0
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable[b] = None
            else:
                self.free.append(b)

    def _block_key(self, seq: int, j: int) -> tuple:
        prev = self.keys[seq][j - 1] if j else ()
        toks = tuple(self.tokens[seq][j * self.B:(j + 1) * self.B])
        return (prev, toks)

    # ----------------------------------------------------------- sequences
    def add_seq(self, seq: int, prompt: Optional[Sequence[int]] = None) -> int:
        """Create a sequence; with prefix caching and a prompt, take over the
        cached blocks of its longest cached whole-block prefix (leaving at
        least one token).  Returns the number of prompt tokens covered."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq], self.lens[seq], self.tokens[seq], self.keys[seq] = [], 0, [], []
        if not (self.prefix_cache and prompt):
            return 0
        prompt = [int(t) for t in prompt]
        prev: tuple = ()
        hit: List[int] = []
        keys: List[tuple] = []
        for j in range((len(prompt) - 1) // self.B):  # leave >= 1 token to compute
            key = (prev, tuple(prompt[j * self.B:(j + 1) * self.B]))
            b = self.cache.get(key)
            if b is None:
                break
            hit.append(b)
            keys.append(key)
            prev = key
        for b in hit:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
        n = len(hit) * self.B
        self.tables[seq] = hit
        self.lens[seq] = n
        self.tokens[seq] = prompt[:n]
        self.keys[seq] = keys
        return n

    def blocks_needed(self, seq: int, n: int) -> int:
        L, B = self.lens[seq], self.B
        need = -(-(L + n) // B) - (-(-L // B))
        if n > 0 and L % B and self.ref[self.tables[seq][-1]] > 1:
            need += 1  # private copy of the shared, partly filled last block
        return need

    def append(self, seq: int, n: int, tokens: Optional[Sequence[int]] = None) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Reserve slots for n new tokens; returns (slots, copy pairs)."""
        if self.prefix_cache and (tokens is None or len(tokens) != n):
            raise ValueError("prefix caching needs the token ids")
        if self.blocks_needed(seq, n) > self.num_free():
            raise OutOfBlocks(f"sequence {seq} needs {self.blocks_needed(seq, n)} blocks")
        table, B = self.tables[seq], self.B
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for i in range(n):
            pos = self.lens[seq]
            j, off = divmod(pos, B)
            if j == len(table):
                table.append(self._allocate())
            elif self.ref[table[j]] > 1:
                nb = self._allocate()
                pairs.append((table[j], nb))
                self._release(table[j])
                table[j] = nb
            slots.append(table[j] * B + off)
            self.lens[seq] += 1
            if self.prefix_cache:
                self.tokens[seq].append(int(tokens[i]))
                if off == B - 1:
                    key = self._block_key(seq, j)
                    self.keys[seq].append(key)
                    if key not in self.cache:
                        self.cache[key] = table[j]
                        self.key_of[table[j]] = key
        return slots, pairs

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (reference counts + 1)."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        for b in self.tables[parent]:
            self.ref[b] += 1
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        self.tokens[child] = list(self.tokens[parent])
        self.keys[child] = list(self.keys[parent])

    def free_seq(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]
        del self.tokens[seq]
        del self.keys[seq]

    # ----------------------------------------------------------- swapping
    def swap_out(self, seq: int, host: "BlockManagerModel") -> List[Tuple[int, int]]:
        """Move a sequence to the host manager; returns (device, host) pairs."""
        table = self.tables[seq]
        if host.num_free() < len(table):
            raise OutOfBlocks("host swap space full")
        host.tables[seq], host.lens[seq], host.tokens[seq] = [], self.lens[seq], list(self.tokens[seq])
        host.keys[seq] = list(self.keys[seq])
        pairs = []
        for b in table:
            hb = host._allocate()
            host.tables[seq].append(hb)
            pairs.append((b, hb))
        self.free_seq(seq)
        return pairs

    def swap_in(self, seq: int, host: "BlockManagerModel") -> List[Tuple[int, int]]:
        """Bring a sequence back from the host manager; returns (host, device) pairs."""
        htable = host.tables[seq]
        if self.num_free() < len(htable):
            raise OutOfBlocks("not enough device blocks to swap in")
        self.tables[seq], self.lens[seq], self.tokens[seq] = [], host.lens[seq], list(host.tokens[seq])
        self.keys[seq] = list(host.keys[seq])
        pairs = []
        for hb in htable:
            b = self._allocate()
            self.tables[seq].append(b)
            pairs.append((hb, b))
        host.free_seq(seq)
        return pairs

    # ----------------------------------------------------------- export
    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        return self.lens[seq]

    def block_tables(self, seqs: Sequence[int], width: int) -> Tuple[List[List[int]], List[int]]:
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if len(t) > width:
                raise ValueError("table wider than the requested width")
            rows.append(t + [-1] * (width - len(t)))
            lens.append(self.lens[s])
        return rows, lens
