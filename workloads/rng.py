"""Seeded, thread-parallel draws of N(0, 1) float32 values.

Large pools (several GB) are filled chunk by chunk.  Chunk ``c`` of a stream
named ``tag`` always uses the generator seeded by ``SeedSequence(seed,
spawn_key=(tag, c))``, so the values depend only on (seed, tag, size) and not
on how many threads run the fill.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _tag_key(tag: str) -> int:
    return zlib.crc32(tag.encode())


def normal_f32(seed: int, tag: str, n: int) -> np.ndarray:
    """``n`` float32 draws from N(0, 1) for stream ``tag`` of ``seed``."""
    return normal_encoded(seed, tag, n, np.float32, None)


def normal_encoded(seed: int, tag: str, n: int, out_dtype, encode) -> np.ndarray:
    """``n`` N(0, 1) draws of stream ``tag``, each chunk passed through ``encode``.

    ``encode`` maps a float32 chunk to the stored representation (or is None
    to keep float32); the draws are identical to ``normal_f32``'s.
    """
    out = np.empty(n, dtype=out_dtype)
    key = _tag_key(tag)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(key, c)))
        if encode is None:
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
        else:
            out[lo:hi] = encode(g.standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(min(_threads(), nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out
