"""CPU oracle for the paged decode-attention path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the entry module's smoke
check and the benchmark's CPU-baseline leg may import or run anything in
this package; the GPU library and its Python binding never do.  The oracle
shares no code with the GPU path: it is plain float64 numpy, written from
the definition of paged attention, and every function is pinned by CPU tests
to closed forms, invariants, a library routine, brute force on tiny inputs
and the pages' own block-table layouts.
"""
from .paged_attention import (
    append_decode,
    attention,
    blocks_held,
    copy_blocks,
    logical_kv,
    merge_partials,
    newest_token_slots,
    paged_decode,
    partial_attention,
    reshape_and_cache,
    swap_blocks,
    token_location,
    widen,
)
from .prefill import causal_rows, paged_prefill

__all__ = [
    "append_decode",
    "attention",
    "causal_rows",
    "blocks_held",
    "copy_blocks",
    "logical_kv",
    "merge_partials",
    "newest_token_slots",
    "paged_decode",
    "paged_prefill",
    "partial_attention",
    "reshape_and_cache",
    "swap_blocks",
    "token_location",
    "widen",
]
