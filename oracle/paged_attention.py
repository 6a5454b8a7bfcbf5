"""Plain CPU oracle for paged decode attention, KV-cache append and block copy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's CPU-baseline leg may import or call this module.
The GPU library never uses it, and it shares no code with the GPU library:
it imports nothing but numpy.

What is computed, and where the pages define it
------------------------------------------------
Page "PagedAttention - Efficient Memory Management for LLM Serving with vLLM"
(irregular6612.github.io), section "Method (PagedAttention + vLLM)": the KV
cache is cut into fixed-size blocks of B tokens; attention walks the block
table, gathers the sequence's non-contiguous blocks and computes
softmax(Q K^T) V.  The block table maps a sequence's logical block number to
a physical block number.  Same page, glossary: logical blocks are the
sequence's own order, physical blocks are positions in the GPU pool.
Page "LLM Inference 8: PagedAttention" (velog.io), section "PagedAttention":
the block table is consulted to find where each part of the cache lives
(its example maps logical 0, 1, 2 to physical 4, 1, 7).

The attention result has a plain definition, so the oracle is that
definition written out in float64: rebuild the sequence's contiguous K and V
by walking its block table, then softmax(scale * K q) V.  It is not a
re-enactment of any kernel: no tiling, no online softmax, no partitions.

Readings where the pages are silent (each also listed in the design notes):
* scale: the pages write softmax(Q K^T) V with no scale; the scale is an
  explicit argument (1/sqrt(D) in the workloads).
* cache layout: [num_blocks, H, B, D] for both K and V.
* slot convention: slot = physical_block * B + offset; negative = skip.
* blocks per sequence: ceil(n / B) (the page on vLLM PagedAttention and
  continuous batching, tech.blogsailing.com, section 4, computes the blocks a
  sequence needs this way); only the last block may be partly filled.
* a context length of 0 yields a zero output.
* storage: f32, f16 or bf16 (bf16 as raw uint16 bit patterns); stored values
  are read exactly and widened to float64.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Reading stored values
# ---------------------------------------------------------------------------


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every stored element.

    f32 and f16 widen exactly through numpy casts.  A bf16 element is the top
    half of a float32 bit pattern: shifting its 16 bits up by 16 gives that
    float32 exactly.
    """
    with np.errstate(invalid="ignore"):  # NaN canaries widen to NaN
        if dtype in ("f32", "f16"):
            return np.asarray(a).astype(np.float64)
        if dtype == "bf16":
            bits = np.asarray(a).astype(np.uint32) << np.uint32(16)
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Block-table walk (logical -> physical)
# ---------------------------------------------------------------------------


def blocks_held(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` tokens occupies: ceil(n / B)."""
    return -(-int(num_tokens) // int(block_size))


def token_location(table_row: np.ndarray, t: int, block_size: int) -> tuple:
    """(physical block, offset) of logical token ``t``: block t // B of the
    sequence, looked up in its block table, at offset t % B."""
    j, off = divmod(int(t), int(block_size))
    return int(table_row[j]), off


def logical_kv(cache: np.ndarray, table_row: np.ndarray, ctx: int) -> np.ndarray:
    """The sequence's first ``ctx`` tokens as a contiguous [H, ctx, D] array.

    Walks logical blocks 0 .. ceil(ctx / B) - 1, takes each one's physical
    block from the table, lays them end to end along the token axis and cuts
    the result at ``ctx`` (only the last block may be partly filled).  Table
    entries past the last needed block and slots past ``ctx`` are never read.
    """
    _, H, B, D = cache.shape
    nb = blocks_held(ctx, B)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and (phys.min() < 0 or phys.max() >= cache.shape[0]):
        raise IndexError("block table entry outside the pool")
    blocks = cache[phys]  # [nb, H, B, D] in logical order
    return blocks.transpose(1, 0, 2, 3).reshape(H, nb * B, D)[:, :ctx, :]


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one head, float64.

    q [D], K [n, D], V [n, D].  Subtracting the maximum score before
    exponentiating leaves the softmax unchanged and keeps exp finite.
    """
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype) -> np.ndarray:
    """Single-query attention of every (sequence, head) over its paged context.

    q [S, H, D]; k_cache, v_cache [N, Hk, B, D]; block_tables int [S, W];
    context_lens int [S].  Returns float64 [S, H, D].

    Hk may be smaller than H (grouped-query attention, named in the
    PagedAttention digest's related work as a way to shrink the KV cache):
    consecutive groups of G = H / Hk query heads share one K/V head, query
    head h reading K/V head h // G.  Hk = H is ordinary multi-head attention.
    """
    S, H, D = q.shape
    Hk = k_cache.shape[1]
    if H % Hk:
        raise ValueError(f"{H} query heads cannot be grouped over {Hk} K/V heads")
    G = H // Hk
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        ctx = int(context_lens[s])
        if ctx <= 0:
            continue
        K = widen(logical_kv(k_cache, block_tables[s], ctx), dtype)
        V = widen(logical_kv(v_cache, block_tables[s], ctx), dtype)
        qs = widen(q[s], dtype)
        for h in range(H):
            out[s, h] = attention(qs[h], K[h // G], V[h // G], scale)
    return out


# ---------------------------------------------------------------------------
# Split over KV partitions: partial results and their merge
# ---------------------------------------------------------------------------


def partial_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Unnormalised attention over one slice of the context.

    Returns (m, l, o): m = max score, l = sum_t exp(s_t - m),
    o = sum_t exp(s_t - m) V_t.  attention() over the slice equals o / l.
    """
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ V


def merge_partials(parts) -> np.ndarray:
    """Combine (m, l, o) partials of disjoint slices into the full attention.

    With M the largest m, every slice's terms exp(s_t - m_p) are rescaled by
    exp(m_p - M) so all share the reference M; the full softmax numerator and
    denominator are then the sums over slices.
    """
    M = max(m for m, _, _ in parts)
    L = sum(np.exp(m - M) * l for m, l, _ in parts)
    O = sum(np.exp(m - M) * o for m, _, o in parts)
    return O / L


# ---------------------------------------------------------------------------
# Cache updates (pure data movement, on copies of the pools)
# ---------------------------------------------------------------------------


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Write token i's K and V rows (all heads) into slot ``slot_mapping[i]``.

    Page "LLM Inference 8: PagedAttention" (velog.io), section on how it
    works: a new token's key and value are stored in the sequence's current
    block, and a new physical block is taken when the current one is full;
    the PagedAttention digest's Method section adds that blocks are
    allocated only as tokens arrive.  Slot = block * B + offset; a negative
    slot is skipped.  Returns new pools; the inputs are not modified.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    N, _, B, _ = kc.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if live.size != np.unique(live).size:
        raise ValueError("duplicate slots")
    if live.size and live.max() >= N * B:
        raise IndexError("slot outside the pool")
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, off = divmod(int(slot), B)
        kc[b, :, off, :] = key[i]
        vc[b, :, off, :] = value[i]
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs):
    """Copy-on-write duplication: physical block dst becomes a copy of src.

    PagedAttention digest, Method: under parallel sampling or beam search the
    samples share the prompt's physical blocks, and only the block that is
    written at the branch point is copied.  The page on vLLM PagedAttention
    and continuous batching, section 2, describes the sharing through
    reference counts.  Every pair copies one whole block (all heads, slots
    and channels) of K and of V.  Destinations must be distinct and must not
    be sources.  Returns new pools.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if pr.size:
        src, dst = pr[:, 0], pr[:, 1]
        if np.unique(dst).size != dst.size:
            raise ValueError("duplicate destination blocks")
        if np.intersect1d(src, dst).size:
            raise ValueError("a block is both a source and a destination")
        if pr.min() < 0 or pr.max() >= kc.shape[0]:
            raise IndexError("block id outside the pool")
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
    return kc, vc


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Move whole blocks between two pools (swapping).

    PagedAttention digest, Method (scheduling) and glossary: under memory
    pressure a preempted request's KV blocks are moved to CPU RAM and moved
    back when it resumes (the page on vLLM PagedAttention and continuous
    batching, section 3, names the same swap space).  For every (src, dst)
    pair, block dst of the destination pools becomes block src of the source
    pools: all heads, slots and channels of K and of V, bit for bit.  The
    pools may differ in their number of blocks (a host swap space is sized on
    its own); destinations must be distinct.  Returns new destination pools.
    """
    kd, vd = dst_k.copy(), dst_v.copy()
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if pr.size:
        src, dst = pr[:, 0], pr[:, 1]
        if np.unique(dst).size != dst.size:
            raise ValueError("duplicate destination blocks")
        if src.min() < 0 or src.max() >= src_k.shape[0] or dst.min() < 0 or dst.max() >= kd.shape[0]:
            raise IndexError("block id outside its pool")
        if src_k.shape[1:] != kd.shape[1:]:
            raise ValueError("pools disagree on heads, block size or head_dim")
        kd[dst] = src_k[src]
        vd[dst] = src_v[src]
    return kd, vd


# ---------------------------------------------------------------------------
# One decode step: store each sequence's newest token, then attend
# ---------------------------------------------------------------------------


def newest_token_slots(block_tables, context_lens, block_size):
    """Slot of every sequence's newest token (position ctx - 1): block
    (ctx - 1) // B of its table at offset (ctx - 1) % B; -1 when ctx <= 0."""
    out = np.full(len(context_lens), -1, dtype=np.int64)
    for s, ctx in enumerate(context_lens):
        if ctx > 0:
            b, off = token_location(block_tables[s], int(ctx) - 1, block_size)
            out[s] = b * block_size + off
    return out


def append_decode(q, key, value, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """The newest token's rows (key, value [S, H, D]) stored at their slots,
    then paged decode over the updated pools.  Returns (out, k_cache', v_cache')."""
    B = k_cache.shape[2]
    slots = newest_token_slots(block_tables, context_lens, B)
    kc, vc = reshape_and_cache(key, value, k_cache, v_cache, slots)
    return paged_decode(q, kc, vc, block_tables, context_lens, scale, dtype), kc, vc
