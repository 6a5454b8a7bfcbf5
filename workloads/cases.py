"""Seeded synthetic workloads for paged decode attention.

Each ``Case`` holds, in storage encoding (see ``storage.py``):

* ``q``            [S, H, D]      one query token per sequence
* ``k_cache``      [N, H, B, D]   physical key blocks (state before ``steps``)
* ``v_cache``      [N, H, B, D]   physical value blocks
* ``block_tables`` int32 [S, W]   logical -> physical block, padded with -1
* ``context_lens`` int32 [S]      tokens each query attends to (after steps)
* ``steps``        cache updates to apply, in order, before the decode:
  ``AppendStep`` (new K/V rows written at slot-mapped positions) and
  ``CopyStep`` (copy-on-write block duplication).

Pool slots that hold no valid token carry NaN canaries.  The recipes follow
the workload shapes of the PagedAttention pages: LLaMA-7B / OPT-13B /
OPT-175B-shaped decode layers, chat-like length mixes standing in for the
ShareGPT traces (which are not available), and parallel sampling with a
shared prompt.  No attention arithmetic happens here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Union

import numpy as np

from .blockpool import BlockPool, SeqBlocks, append_tokens, cow_last_block, fork, tables_array
from .rng import normal_encoded
from .storage import NP_STORAGE, canary_fill, to_storage

BASE_SEED = 322


@dataclass
class AppendStep:
    key: np.ndarray  # [T, H, D] storage
    value: np.ndarray  # [T, H, D] storage
    slot_mapping: np.ndarray  # int64 [T]


@dataclass
class CopyStep:
    pairs: np.ndarray  # int64 [n, 2] of (src, dst)


Step = Union[AppendStep, CopyStep]


@dataclass
class Case:
    name: str
    dtype: str
    num_heads: int  # query heads
    head_dim: int
    block_size: int
    num_blocks: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    scale: float
    steps: List[Step] = field(default_factory=list)
    meta: dict = field(default_factory=dict)
    # Prefill cases: int32 [S + 1]; sequence s owns query rows
    # query_start[s] .. query_start[s + 1] - 1 of q (packed [T, H, D]).
    # None for decode cases (one query row per sequence).
    query_start: Optional[np.ndarray] = None

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        """Query rows: one per sequence for decode, the packed chunks for prefill."""
        return int(self.q.shape[0])

    @property
    def query_lens(self) -> np.ndarray:
        if self.query_start is None:
            return np.ones(self.num_seqs, dtype=np.int64)
        return np.diff(self.query_start).astype(np.int64)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return int(self.q.dtype.itemsize)


def normal_storage(seed: int, tag: str, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    return normal_encoded(seed, tag, n, NP_STORAGE[dtype], lambda x: to_storage(x, dtype)).reshape(shape)


def _fill_history(cache: np.ndarray, seqs: Sequence[SeqBlocks], hist: Sequence[int], seed: int, tag: str, dtype: str) -> None:
    """Write N(0, 1) values into the first ``hist[i]`` token slots of every sequence.

    Full blocks are filled in chunks of whole blocks; each sequence's final
    partially filled block gets only its filled slots, the rest keep their
    canaries.  Values are drawn per physical block in allocation order.
    """
    _, H, B, D = cache.shape
    full: List[int] = []
    partial: List[tuple] = []
    for s, n in zip(seqs, hist):
        nfull, rem = divmod(int(n), B)
        full.extend(s.table[:nfull])
        if rem:
            partial.append((s.table[nfull], rem))
    chunk = max(1, (1 << 26) // (H * B * D))
    for c0 in range(0, len(full), chunk):
        ids = np.asarray(full[c0 : c0 + chunk], dtype=np.int64)
        cache[ids] = normal_storage(seed, f"{tag}/full/{c0}", (len(ids), H, B, D), dtype)
    if partial:
        total = sum(r for _, r in partial)
        vals = normal_storage(seed, f"{tag}/partial", (H, total, D), dtype)
        o = 0
        for b, r in partial:
            cache[b, :, :r, :] = vals[:, o : o + r, :]
            o += r


def _paged_case(name, dtype, H, D, B, N, ctx, seed, perm, n_append: int, scale=None, Hk=None) -> Case:
    """Sequences with ``ctx[i] - n_append`` history tokens in a permuted pool and
    ``n_append`` new tokens per sequence written by an append step.  The
    caches hold ``Hk`` K/V heads (default: one per query head)."""
    Hk = H if Hk is None else Hk
    pool = BlockPool(N, B, perm)
    seqs = [SeqBlocks() for _ in ctx]
    hist = [int(c) - n_append for c in ctx]
    assert min(hist) >= 0
    for s, h in zip(seqs, hist):
        append_tokens(pool, s, h)
    k_cache = canary_fill((N, Hk, B, D), dtype)
    v_cache = canary_fill((N, Hk, B, D), dtype)
    _fill_history(k_cache, seqs, hist, seed, "k", dtype)
    _fill_history(v_cache, seqs, hist, seed, "v", dtype)
    steps: List[Step] = []
    if n_append:
        slots: List[int] = []
        for s in seqs:
            sl, pairs = append_tokens(pool, s, n_append)
            assert not pairs
            slots.extend(sl)
        T = len(slots)
        steps.append(
            AppendStep(
                normal_storage(seed, "k_new", (T, Hk, D), dtype),
                normal_storage(seed, "v_new", (T, Hk, D), dtype),
                np.asarray(slots, dtype=np.int64),
            )
        )
    q = normal_storage(seed, "q", (len(ctx), H, D), dtype)
    return Case(
        name=name,
        dtype=dtype,
        num_heads=H,
        head_dim=D,
        block_size=B,
        num_blocks=N,
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=tables_array(seqs),
        context_lens=np.asarray(ctx, dtype=np.int32),
        scale=(1.0 / math.sqrt(D)) if scale is None else scale,
        steps=steps,
        meta={"blocks_used": pool.used},
    )


def _prefill_case(name, dtype, H, D, B, N, prefix, chunk, seed, perm, Hk=None, scale=None) -> Case:
    """Chunked prefill.  Sequence i already holds ``prefix[i]`` tokens in the
    cache (earlier chunks of its prompt, or a cached shared prefix) and brings
    ``chunk[i]`` new prompt tokens.  An append step writes the chunk's K/V
    rows into the sequence's blocks (new blocks only when the current one is
    full); the chunk's queries are packed into q [T, H, D], T = sum(chunk),
    with ``query_start`` [S + 1] marking each sequence's rows.  After the
    step the context length is prefix + chunk."""
    Hk = H if Hk is None else Hk
    prefix = [int(p) for p in prefix]
    chunk = [int(c) for c in chunk]
    assert len(prefix) == len(chunk) and min(chunk) >= 1 and min(prefix) >= 0
    pool = BlockPool(N, B, perm)
    seqs = [SeqBlocks() for _ in prefix]
    for s, p in zip(seqs, prefix):
        append_tokens(pool, s, p)
    k_cache = canary_fill((N, Hk, B, D), dtype)
    v_cache = canary_fill((N, Hk, B, D), dtype)
    _fill_history(k_cache, seqs, prefix, seed, "k", dtype)
    _fill_history(v_cache, seqs, prefix, seed, "v", dtype)
    slots: List[int] = []
    for s, n in zip(seqs, chunk):
        sl, pairs = append_tokens(pool, s, n)
        assert not pairs
        slots.extend(sl)
    T = len(slots)
    step = AppendStep(
        normal_storage(seed, "k_chunk", (T, Hk, D), dtype),
        normal_storage(seed, "v_chunk", (T, Hk, D), dtype),
        np.asarray(slots, dtype=np.int64),
    )
    qs = np.zeros(len(chunk) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(chunk)
    return Case(
        name=name,
        dtype=dtype,
        num_heads=H,
        head_dim=D,
        block_size=B,
        num_blocks=N,
        q=normal_storage(seed, "q_chunk", (T, H, D), dtype),
        k_cache=k_cache,
        v_cache=v_cache,
        block_tables=tables_array(seqs),
        context_lens=np.asarray([p + c for p, c in zip(prefix, chunk)], dtype=np.int32),
        scale=(1.0 / math.sqrt(D)) if scale is None else scale,
        steps=[step],
        meta={"blocks_used": pool.used, "prefix": np.asarray(prefix), "chunk": np.asarray(chunk)},
        query_start=qs,
    )


# --------------------------------------------------------------------------
# The decode workloads: a tiny fp32 case and four model-shaped layers.
# --------------------------------------------------------------------------

def tiny_f32() -> Case:
    seed = BASE_SEED + 1
    rng = np.random.default_rng(seed)
    perm = rng.permutation(16)
    return _paged_case("tiny-f32", "f32", 1, 8, 4, 16, [5, 16, 37], seed, perm, 0, scale=1.0 / math.sqrt(8.0))


def llama7b_decode(num_seqs: int = 64, n_append: int = 0) -> Case:
    """LLaMA-7B-shaped decode layer.  With ``n_append`` = 1 the last context
    token of every sequence is written by an append step (a serving decode
    step: store the current token's K/V, then attend)."""
    seed = BASE_SEED + 2
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 2049, 64)[:num_seqs]
    perm = rng.permutation(8192)
    return _paged_case("llama7b-decode", "f16", 32, 128, 16, 8192, ctx, seed, perm, n_append)


def opt13b_context_lengths() -> np.ndarray:
    rng = np.random.default_rng(BASE_SEED + 3)
    return np.clip(np.round(rng.lognormal(math.log(300.0), 0.9, 256)), 16, 2048).astype(np.int64)


def opt13b_decode() -> Case:
    seed = BASE_SEED + 3
    ctx = opt13b_context_lengths()
    rng = np.random.default_rng([seed, 1])
    perm = rng.permutation(16384)
    return _paged_case("opt13b-decode", "f16", 40, 128, 16, 16384, ctx, seed, perm, 1)


def opt175b_decode(num_heads: int = 96, n_append: int = 0) -> Case:
    seed = BASE_SEED + 5
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1024, 2049, 128)
    perm = rng.permutation(16384)
    return _paged_case("opt175b-decode", "bf16", num_heads, 128, 16, 16384, ctx, seed, perm, n_append)


def parallel_sampling(
    block_size: int = 16,
    num_prompts: int = 64,
    samples: int = 4,
    prompt_len: int = 500,
    num_heads: int = 40,
    head_dim: int = 128,
    pool_tokens: int = 262144,
    dtype: str = "f16",
    max_suffix: int = 256,
    num_kv_heads: Optional[int] = None,
) -> Case:
    """Parallel sampling with copy-on-write of the shared partial prompt block.

    Order of cache updates: the prompt K/V of every prompt is appended once;
    each prompt forks into ``samples`` sequences that share all prompt blocks;
    samples 0..n-2 take private copies of the partially filled last prompt
    block (one batched block copy), sample n-1 keeps the original; each sample
    then appends its own suffix tokens; decode attends to prompt + suffix.
    Suffix lengths are uniform in [0, max_suffix]; with the defaults (at most
    64 prompts of at most 4 samples, f16) the draws are those of the
    parallel-sampling workload.  num_kv_heads (a divisor of num_heads, default
    num_heads) gives grouped-query caches.
    """
    seed = BASE_SEED + 4
    D, B = head_dim, block_size
    H = num_heads
    Hk = H if num_kv_heads is None else num_kv_heads
    assert H % Hk == 0
    rng = np.random.default_rng(seed)
    if num_prompts <= 64 and samples <= 4 and max_suffix == 256:
        suffix = rng.integers(0, 257, (64, 4))[:num_prompts, :samples]
    else:
        suffix = np.random.default_rng([seed, samples, max_suffix]).integers(0, max_suffix + 1,
                                                                             (num_prompts, samples))
    N = pool_tokens // B
    perm = np.random.default_rng([seed, B]).permutation(N)
    pool = BlockPool(N, B, perm)
    prompts = [SeqBlocks() for _ in range(num_prompts)]
    prompt_slots: List[int] = []
    for p in prompts:
        sl, pairs = append_tokens(pool, p, prompt_len)
        assert not pairs
        prompt_slots.extend(sl)
    prompt_blocks = pool.used
    kids: List[SeqBlocks] = []
    pairs: List[tuple] = []
    for p in prompts:
        ks = fork(pool, p, samples)
        for k in ks[:-1]:
            pairs.extend(cow_last_block(pool, k))
        kids.extend(ks)
    suffix_slots: List[int] = []
    for i, k in enumerate(kids):
        sl, pr = append_tokens(pool, k, int(suffix.reshape(-1)[i]))
        assert not pr  # the only shared block was copied at the fork
        suffix_slots.extend(sl)
    ctx = np.asarray([k.length for k in kids], dtype=np.int32)
    no_share = sum(math.ceil(int(c) / B) for c in ctx)
    T0, T1 = len(prompt_slots), len(suffix_slots)
    steps: List[Step] = [
        AppendStep(
            normal_storage(seed, f"kp/{B}", (T0, Hk, D), dtype),
            normal_storage(seed, f"vp/{B}", (T0, Hk, D), dtype),
            np.asarray(prompt_slots, dtype=np.int64),
        ),
        CopyStep(np.asarray(pairs, dtype=np.int64).reshape(-1, 2)),
        AppendStep(
            normal_storage(seed, f"ks/{B}", (T1, Hk, D), dtype),
            normal_storage(seed, f"vs/{B}", (T1, Hk, D), dtype),
            np.asarray(suffix_slots, dtype=np.int64),
        ),
    ]
    return Case(
        name=f"parallel-sampling-B{B}" + ("" if dtype == "f16" else f"-{dtype}") + ("" if Hk == H else f"-Hk{Hk}"),
        dtype=dtype,
        num_heads=H,
        head_dim=D,
        block_size=B,
        num_blocks=N,
        q=normal_storage(seed, f"q/{B}", (len(kids), H, D), dtype),
        k_cache=canary_fill((N, Hk, B, D), dtype),
        v_cache=canary_fill((N, Hk, B, D), dtype),
        block_tables=tables_array(kids),
        context_lens=ctx,
        scale=1.0 / math.sqrt(D),
        steps=steps,
        meta={
            "blocks_used": pool.used,
            "prompt_blocks": prompt_blocks,
            "blocks_without_sharing": no_share,
            "kv_memory_saved": 1.0 - pool.used / no_share,
            "samples": samples,
        },
    )


GQA_NAMES = {
    "llama3-8b": "llama3-8b-gqa-decode: 64 seqs ctx U[128,2048], H=32 query / 8 K/V heads, D=128, f16, B=16",
    "llama2-70b-tp8": "llama2-70b-gqa-tp8-share: 128 seqs ctx U[512,4096], H=8 query / 1 K/V head, D=128, bf16, B=16",
}


def gqa_config(kind: str = "llama3-8b", n_append: int = 0) -> Case:
    """Grouped-query decode layers (query heads share K/V heads).

    llama3-8b: the LLaMA-7B-shaped decode batch with 32 query heads over
    8 K/V heads (groups of 4).  llama2-70b-tp8: one tensor-parallel rank's
    share of a 64-query / 8-K/V-head layer (8 query heads over 1 K/V head,
    groups of 8), 128 sequences of 512..4096 tokens.
    """
    if kind == "llama3-8b":
        seed = BASE_SEED + 6
        rng = np.random.default_rng(seed)
        ctx = rng.integers(128, 2049, 64)
        perm = rng.permutation(8192)
        return _paged_case("gqa-llama3-8b", "f16", 32, 128, 16, 8192, ctx, seed, perm, n_append, Hk=8)
    if kind == "llama2-70b-tp8":
        seed = BASE_SEED + 7
        rng = np.random.default_rng(seed)
        ctx = rng.integers(512, 4097, 128)
        perm = rng.permutation(32768)
        return _paged_case("gqa-llama2-70b-tp8", "bf16", 8, 128, 16, 32768, ctx, seed, perm, n_append, Hk=1)
    raise ValueError(kind)


PREFILL_NAMES = {
    "llama7b": "llama7b-chunked-prefill: 16 seqs, 512-token chunks over cached prefixes U[0,1536], H=32, D=128, f16, B=16",
    "llama3-8b": "llama3-8b-chunked-prefill: 16 seqs, 512-token chunks over cached prefixes U[0,1536], 32 query / 8 K/V heads, D=128, f16, B=16",
    "prompts": "llama7b-prompt-prefill: 32 whole prompts, lognormal(300, 0.9) lengths clipped [16, 2048], H=32, D=128, bf16, B=16",
}


def prefill_config(kind: str = "llama7b") -> Case:
    """Prefill workloads (the step before decode).

    llama7b / llama3-8b: one chunked-prefill step.  Each of 16 sequences has
    a cached prefix of U[0, 1536] tokens (earlier chunks) and brings a
    512-token chunk; the LLaMA-7B-shaped layer (32 heads) and the
    LLaMA-3-8B-shaped one (32 query over 8 K/V heads).
    prompts: whole-prompt prefill of 32 prompts with the chat-like lognormal
    length mix of the OPT-13B-shaped batch (no cached prefix), bf16.
    """
    if kind in ("llama7b", "llama3-8b"):
        seed = BASE_SEED + 8
        rng = np.random.default_rng(seed)
        prefix = rng.integers(0, 1537, 16)
        perm = rng.permutation(4096)
        Hk = 32 if kind == "llama7b" else 8
        return _prefill_case(f"prefill-{kind}", "f16", 32, 128, 16, 4096, prefix, [512] * 16, seed, perm, Hk=Hk)
    if kind == "prompts":
        seed = BASE_SEED + 9
        rng = np.random.default_rng(seed)
        lens = np.clip(np.round(rng.lognormal(math.log(300.0), 0.9, 32)), 16, 2048).astype(np.int64)
        perm = rng.permutation(4096)
        return _prefill_case("prefill-prompts", "bf16", 32, 128, 16, 4096, [0] * 32, lens, seed, perm)
    raise ValueError(kind)


def random_prefill_case(
    seed: int,
    prefix: Sequence[int],
    chunk: Sequence[int],
    num_heads: int,
    head_dim: int,
    block_size: int,
    dtype: str,
    num_kv_heads: Optional[int] = None,
    spare_blocks: int = 3,
) -> Case:
    """Small chunked-prefill case for parity tests (seeded, permuted pool)."""
    rng = np.random.default_rng([BASE_SEED, 77, seed])
    need = sum(-(-(int(p) + int(c)) // block_size) for p, c in zip(prefix, chunk))
    N = need + spare_blocks
    perm = rng.permutation(N)
    return _prefill_case(f"prefill-random-{seed}", dtype, num_heads, head_dim, block_size, N, prefix, chunk,
                         BASE_SEED * 1000 + seed, perm, Hk=num_kv_heads)


# --------------------------------------------------------------------------
# Random small cases for parity sweeps.
# --------------------------------------------------------------------------


def random_case(
    seed: int,
    num_seqs: int,
    num_heads: int,
    head_dim: int,
    block_size: int,
    dtype: str,
    ctx: Optional[Sequence[int]] = None,
    ctx_range=(1, 64),
    spare_blocks: int = 3,
    n_append: int = 0,
    scale: Optional[float] = None,
    num_kv_heads: Optional[int] = None,
) -> Case:
    """A small paged case with a seeded random physical placement."""
    rng = np.random.default_rng([BASE_SEED, seed])
    if ctx is None:
        ctx = rng.integers(ctx_range[0], ctx_range[1] + 1, num_seqs)
    ctx = [int(c) for c in ctx]
    need = sum(max(0, math.ceil(c / block_size)) for c in ctx)
    N = need + spare_blocks
    perm = rng.permutation(N)
    return _paged_case(
        f"random-{seed}", dtype, num_heads, head_dim, block_size, N, ctx, seed * 7919 + 17, perm, n_append,
        scale=scale, Hk=num_kv_heads,
    )
