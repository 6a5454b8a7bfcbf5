"""Plain CPU oracle for paged prefill attention (prompt and chunked prefill).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's CPU-baseline leg may import or call this module.
The GPU library never uses it and shares no code with it; it imports numpy
and the decode oracle's block-table walk, nothing else.

What is computed, and where the pages define it
------------------------------------------------
Before a sequence decodes, its prompt is run through the model once
(prefill).  Page "vLLM PagedAttention and continuous batching architecture"
(tech.blogsailing.com), section 3: the scheduler prefills newly arrived
requests in the same forward pass as the sequences that are decoding, and
section 5 (tuning): with chunked prefill a long prompt's prefill tokens are
split into fixed-size chunks so decoding batches are not stalled.  Page
"KV cache and PagedAttention: LLM inference speed and GPU throughput"
(allinfo.ai.kr), key insights: chunked prefill fills the step with decode
requests first and spends the rest on prefill chunks; with prefix caching,
requests that share a prefix point at the same physical blocks and skip its
prefill.  Same page, introduction: in autoregressive generation every token
attends to the tokens before it, whose keys and values the KV cache holds.

So one prefill call takes, per sequence, a chunk of n new prompt tokens
whose keys and values are already in the paged cache (written by the append
step), after ctx - n earlier tokens (earlier chunks, or a cached prefix).
Reading taken where the pages are silent: the chunk occupies positions
ctx - n .. ctx - 1 of the context, and the query at position p attends to
the tokens at positions 0 .. p (causal, the decoder-only reading of "attends
to the tokens before it", itself included).  n = ctx is a whole-prompt
prefill; n = 1 is one decode query.  The result has a plain definition, so
the oracle is that definition in float64: gather the sequence's K and V
through its block table (the decode oracle's walk), then for every query row
softmax over its allowed keys.  No tiling, no online softmax.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attention, logical_kv, widen


def causal_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, first_pos: int) -> np.ndarray:
    """Attention rows for queries at positions first_pos .. first_pos + n - 1.

    Q [n, D]; K, V [ctx, D] with ctx >= first_pos + n.  Row i attends to the
    keys at positions 0 .. first_pos + i.
    """
    n = Q.shape[0]
    out = np.empty((n, Q.shape[1]), dtype=np.float64)
    for i in range(n):
        p = first_pos + i
        out[i] = attention(Q[i], K[: p + 1], V[: p + 1], scale)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype) -> np.ndarray:
    """Causal attention of every sequence's chunk over its paged context.

    q [T, H, D] packed query rows; query_start int [S + 1]: sequence s owns
    rows query_start[s] .. query_start[s + 1] - 1 (n_s of them, n_s <=
    context_lens[s]); k_cache, v_cache [N, Hk, B, D] with the chunk's rows
    already written; block_tables int [S, W]; context_lens int [S] (after
    the chunk).  Query head h reads K/V head h // (H / Hk).  Returns float64
    [T, H, D].
    """
    T, H, D = q.shape
    Hk = k_cache.shape[1]
    if H % Hk:
        raise ValueError(f"{H} query heads cannot be grouped over {Hk} K/V heads")
    G = H // Hk
    qs = np.asarray(query_start, dtype=np.int64)
    if qs[0] != 0 or qs[-1] != T or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must rise from 0 to the number of query rows")
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in range(len(context_lens)):
        r0, r1 = int(qs[s]), int(qs[s + 1])
        n, ctx = r1 - r0, int(context_lens[s])
        if n == 0:
            continue
        if n > ctx:
            raise ValueError("a chunk longer than its context")
        K = widen(logical_kv(k_cache, block_tables[s], ctx), dtype)
        V = widen(logical_kv(v_cache, block_tables[s], ctx), dtype)
        Qs = widen(q[r0:r1], dtype)  # [n, H, D]
        for h in range(H):
            out[r0:r1, h] = causal_rows(Qs[:, h], K[h // G], V[h // G], scale, ctx - n)
    return out
