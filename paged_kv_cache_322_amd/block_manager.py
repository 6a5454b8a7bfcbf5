"""ctypes binding of libpa's host-side block manager (include/pa_block_manager.h).

Argument marshalling only: every decision (free list, reference counts,
copy-on-write, prefix caching, swap bookkeeping) is taken by the C++
manager in the library.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import PagedAttentionError, lib

_p = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64
# Array arguments are passed as raw addresses (numpy's ctypes.data_as goes
# through ctypes.cast, which costs ~0.4 ms per call).
_I32P = _I64P = ctypes.c_void_p

lib.pa_bm_create.restype = _p
lib.pa_bm_create.argtypes = [_i64, _i32, _I32P, _i32]
lib.pa_bm_destroy.restype = None
lib.pa_bm_destroy.argtypes = [_p]
lib.pa_bm_add_seq.restype = ctypes.c_int
lib.pa_bm_add_seq.argtypes = [_p, _i64, _I32P, _i32, _I32P]
lib.pa_bm_append.restype = ctypes.c_int
lib.pa_bm_append.argtypes = [_p, _i64, _i32, _I32P, _I64P, _I64P, _I32P]
lib.pa_bm_append_batch.restype = ctypes.c_int
lib.pa_bm_append_batch.argtypes = [_p, _I64P, _i32, _I32P, _I64P, _I64P, _I32P, _I32P]
lib.pa_bm_fork.restype = ctypes.c_int
lib.pa_bm_fork.argtypes = [_p, _i64, _i64]
lib.pa_bm_free_seq.restype = ctypes.c_int
lib.pa_bm_free_seq.argtypes = [_p, _i64]
lib.pa_bm_swap_out.restype = ctypes.c_int
lib.pa_bm_swap_out.argtypes = [_p, _p, _i64, _I64P, _i32, _I32P]
lib.pa_bm_swap_in.restype = ctypes.c_int
lib.pa_bm_swap_in.argtypes = [_p, _p, _i64, _I64P, _i32, _I32P]
lib.pa_bm_block_tables.restype = ctypes.c_int
lib.pa_bm_block_tables.argtypes = [_p, _I64P, _i32, _i32, _I32P, _I32P]
for _name, _res, _args in (("pa_bm_num_free", _i64, [_p]), ("pa_bm_seq_len", _i64, [_p, _i64]),
                           ("pa_bm_num_blocks_held", _i32, [_p, _i64]),
                           ("pa_bm_blocks_needed", _i32, [_p, _i64, _i32]),
                           ("pa_bm_ref_count", _i32, [_p, _i32]), ("pa_bm_num_cached", _i64, [_p])):
    getattr(lib, _name).restype = _res
    getattr(lib, _name).argtypes = _args

OUT_OF_BLOCKS = 5  # PA_ERR_OUT_OF_BLOCKS


class OutOfBlocks(PagedAttentionError):
    """Not enough free blocks; the manager is unchanged."""


def _check(status: int, what: str) -> None:
    if status == OUT_OF_BLOCKS:
        raise OutOfBlocks(status, what)
    if status != 0:
        raise PagedAttentionError(status, what)


def _i32_array(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr32(a: Optional[np.ndarray]):
    assert a is None or (a.dtype == np.int32 and a.flags.c_contiguous)
    return None if a is None else a.ctypes.data


def _ptr64(a: Optional[np.ndarray]):
    assert a is None or (a.dtype == np.int64 and a.flags.c_contiguous)
    return None if a is None else a.ctypes.data


class BlockManager:
    """Free list, reference counts, copy-on-write, prefix cache and swap
    bookkeeping of one pool of ``num_blocks`` blocks of ``block_size`` tokens."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None,
                 prefix_cache: bool = False):
        order = None if free_order is None else _i32_array(free_order)
        if order is not None and order.size != num_blocks:
            raise ValueError("free_order must list every block once")
        h = lib.pa_bm_create(int(num_blocks), int(block_size), _ptr32(order), 1 if prefix_cache else 0)
        if not h:
            raise ValueError("invalid block manager arguments (sizes or free order)")
        self._h = ctypes.c_void_p(h)
        self._destroy = lib.pa_bm_destroy  # kept: module globals may be gone when the object dies at exit
        self.num_blocks, self.block_size, self.prefix_cache = int(num_blocks), int(block_size), bool(prefix_cache)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    # sequences
    def add_seq(self, seq: int, prompt: Optional[Sequence[int]] = None) -> int:
        p = None if prompt is None else _i32_array(prompt)
        cached = ctypes.c_int32(0)
        _check(lib.pa_bm_add_seq(self._h, int(seq), _ptr32(p), 0 if p is None else p.size, ctypes.byref(cached)),
               "pa_bm_add_seq")
        return int(cached.value)

    def append(self, seq: int, n: int, tokens: Optional[Sequence[int]] = None) -> Tuple[List[int], List[Tuple[int, int]]]:
        t = None if tokens is None else _i32_array(tokens)
        if t is not None and t.size != n:
            raise ValueError("one token id per appended token")
        slots = np.empty(max(n, 1), dtype=np.int64)
        pair = np.empty(2, dtype=np.int64)
        npairs = ctypes.c_int32(0)
        _check(lib.pa_bm_append(self._h, int(seq), int(n), _ptr32(t), _ptr64(slots), _ptr64(pair),
                                ctypes.byref(npairs)), "pa_bm_append")
        return slots[:n].tolist(), ([(int(pair[0]), int(pair[1]))] if npairs.value else [])

    def append_batch(self, seqs: Sequence[int], tokens: Optional[Sequence[int]] = None):
        """One token for each sequence (a decode step): (slots int64 [S], pairs int64 [k, 2])."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        t = None if tokens is None else _i32_array(tokens)
        slots = np.empty(max(s.size, 1), dtype=np.int64)
        pairs = np.empty((max(s.size, 1), 2), dtype=np.int64)
        npairs, done = ctypes.c_int32(0), ctypes.c_int32(0)
        st = lib.pa_bm_append_batch(self._h, _ptr64(s), s.size, _ptr32(t), _ptr64(slots), _ptr64(pairs),
                                    ctypes.byref(npairs), ctypes.byref(done))
        if st != 0:
            err = OutOfBlocks if st == OUT_OF_BLOCKS else PagedAttentionError
            e = err(st, f"pa_bm_append_batch (stopped after {done.value} of {s.size} sequences)")
            e.done = done.value
            raise e
        return slots[: s.size], pairs[: npairs.value]

    def fork(self, parent: int, child: int) -> None:
        _check(lib.pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_seq(self, seq: int) -> None:
        _check(lib.pa_bm_free_seq(self._h, int(seq)), "pa_bm_free_seq")

    def _move(self, fn, seq, host) -> List[Tuple[int, int]]:
        cap = max(1, self.num_blocks_held(seq) if fn is lib.pa_bm_swap_out else host.num_blocks_held(seq))
        pairs = np.empty((cap, 2), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(fn(self._h, host._h, int(seq), _ptr64(pairs), cap, ctypes.byref(n)), fn.__name__)
        return [(int(a), int(b)) for a, b in pairs[: n.value]]

    def swap_out(self, seq: int, host: "BlockManager") -> List[Tuple[int, int]]:
        """Move ``seq`` to the host manager; returns (device block, host block) pairs."""
        return self._move(lib.pa_bm_swap_out, seq, host)

    def swap_in(self, seq: int, host: "BlockManager") -> List[Tuple[int, int]]:
        """Bring ``seq`` back from the host manager; returns (host block, device block) pairs."""
        return self._move(lib.pa_bm_swap_in, seq, host)

    # queries
    def num_free(self) -> int:
        return int(lib.pa_bm_num_free(self._h))

    def num_cached(self) -> int:
        return int(lib.pa_bm_num_cached(self._h))

    def length(self, seq: int) -> int:
        n = int(lib.pa_bm_seq_len(self._h, int(seq)))
        if n < 0:
            raise KeyError(seq)
        return n

    def num_blocks_held(self, seq: int) -> int:
        n = int(lib.pa_bm_num_blocks_held(self._h, int(seq)))
        if n < 0:
            raise KeyError(seq)
        return n

    def blocks_needed(self, seq: int, n: int) -> int:
        return int(lib.pa_bm_blocks_needed(self._h, int(seq), int(n)))

    def ref_count(self, block: int) -> int:
        return int(lib.pa_bm_ref_count(self._h, int(block)))

    def table(self, seq: int) -> List[int]:
        rows, _ = self.block_tables_array([seq], self.num_blocks_held(seq))
        return rows[0].tolist()

    def block_tables_array(self, seqs: Sequence[int], width: int):
        """int32 [S, width] tables padded with -1, and int32 [S] lengths."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        tables = np.empty((s.size, max(width, 0)), dtype=np.int32)
        lens = np.empty(s.size, dtype=np.int32)
        _check(lib.pa_bm_block_tables(self._h, _ptr64(s), s.size, int(width), _ptr32(tables), _ptr32(lens)),
               "pa_bm_block_tables")
        return tables, lens

    def block_tables(self, seqs: Sequence[int], width: int):
        t, l = self.block_tables_array(seqs, width)
        return t.tolist(), l.tolist()
