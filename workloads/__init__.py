"""Seeded synthetic inputs for paged decode attention.

Shared by the CPU oracle tests and the GPU path's tests and benchmark.  It
holds input generation and host-side block bookkeeping only: no step of the
attention, cache-write or block-copy computation lives here.
"""
from .blockpool import BlockPool, PoolExhausted, SeqBlocks, append_tokens, cow_last_block, fork, tables_array
from .cases import (
    GQA_NAMES,
    PREFILL_NAMES,
    AppendStep,
    Case,
    CopyStep,
    tiny_f32,
    llama7b_decode,
    opt13b_decode,
    opt13b_context_lengths,
    parallel_sampling,
    opt175b_decode,
    gqa_config,
    normal_storage,
    prefill_config,
    random_case,
    random_prefill_case,
)
from .rng import normal_f32
from .storage import CANARY_BITS, DTYPES, ELEM_BYTES, NP_BITS, NP_STORAGE, bits_view, canary_fill, f32_to_bf16_bits, to_storage
