"""Seeded random shapes through the C ABI against the oracle: decode
(multi-head and grouped heads, every dtype, forced and default partitions,
with and without the fused append), sibling groups of forked samples, and
chunked prefill.  Each case is small
enough for the oracle to check every output; together they cross the plan
thresholds, block sizes and ragged tails the hand-written cases pick one at
a time."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import GpuCase, assert_close, assert_pool_equal, log, oracle_decode, oracle_steps, pa

pytestmark = pytest.mark.gpu

HEAD_DIMS = {"f32": [8, 32, 64, 128], "f16": [64, 128, 256], "bf16": [64, 128, 256]}


def _decode_case(seed: int):
    rng = np.random.default_rng([322, 9001, seed])
    dtype = ["f32", "f16", "bf16"][seed % 3]
    D = int(rng.choice(HEAD_DIMS[dtype]))
    B = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hk = int(rng.choice([1, 2, 3]))
    S = int(rng.integers(1, 9))
    ctx = rng.integers(1, 700, S)
    part = int(rng.choice([0, 0, 16, 64, 256]))
    return dtype, D, B, G, Hk, S, ctx, part


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    case, part = random_decode_case(seed)
    dtype = case.dtype
    log(f"seed {seed}: {dtype} D={case.head_dim} B={case.block_size} H={case.num_heads} Hk={case.num_kv_heads} "
        f"part={part} ctx={case.context_lens.tolist()}")
    g = GpuCase(case)
    kc, vc = case.k_cache, case.v_cache
    for i, (kc, vc) in enumerate(oracle_steps(case)):
        g.run_step(i)
        assert_pool_equal(g.kc, kc, dtype, f"seed {seed} K after step {i}")
        assert_pool_equal(g.vc, vc, dtype, f"seed {seed} V after step {i}")
    ref = oracle_decode(case, kc, vc)
    out = g.decode(partition=part, out=torch.empty_like(g.q))
    torch.cuda.synchronize()
    assert_close(out, ref, dtype, f"seed {seed} decode", strict=False)


def random_decode_case(seed: int) -> tuple:
    """(case, forced partition or 0) of random decode seed `seed`."""
    dtype, D, B, G, Hk, S, ctx, part = _decode_case(seed)
    case = wl.random_case(5000 + seed, S, G * Hk, D, B, dtype, ctx=ctx, spare_blocks=4, n_append=1, num_kv_heads=Hk)
    return case, part


def random_prefill_case(seed: int) -> wl.Case:
    rng = np.random.default_rng([322, 9002, seed])
    dtype = ["f16", "bf16"][seed % 2]
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([1, 4, 16, 32, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hk = int(rng.choice([1, 2]))
    S = int(rng.integers(1, 6))
    prefix = rng.integers(0, 400, S).tolist()
    chunk = rng.integers(1, 300, S).tolist()
    return wl.random_prefill_case(7000 + seed, prefix, chunk, G * Hk, D, B, dtype, num_kv_heads=Hk)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    from test_gpu_prefill import check

    case = random_prefill_case(seed)
    log(f"seed {seed}: {case.dtype} D={case.head_dim} B={case.block_size} H={case.num_heads} "
        f"Hk={case.num_kv_heads} ctx={case.context_lens.tolist()} rows={np.diff(case.query_start).tolist()}")
    check(case, strict=False)


def random_siblings_case(seed: int) -> tuple:
    """(case, group size) of random sibling seed `seed`: forked samples of a
    few prompts (copy-on-write of the partly filled last prompt block), with
    a group size that may or may not match the samples per prompt."""
    rng = np.random.default_rng([322, 9003, seed])
    dtype = ["f16", "bf16"][seed % 2]
    D = int(rng.choice([64, 128, 256]))
    B = int(rng.choice([1, 2, 8, 16, 32, 64, 256]))
    samples = int(rng.integers(1, 9))
    prompts = int(rng.integers(1, 5))
    prompt_len = int(rng.integers(1, 400))
    max_suffix = int(rng.integers(0, 200))
    group = int(rng.choice([samples, samples, 2, 3, 16])) if samples >= 2 else int(rng.choice([2, 5]))
    need = prompts * samples * ((prompt_len + max_suffix) // B + 3)
    Hk = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 1, 2, 4]))
    group = max(2, min(16 // G, group))
    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=prompt_len,
                                num_heads=Hk * G, head_dim=D, pool_tokens=max(4096, 2 * need * B), dtype=dtype,
                                max_suffix=max_suffix, num_kv_heads=Hk)
    return case, group


@pytest.mark.parametrize("seed", range(16))
def test_random_siblings(seed):
    case, group = random_siblings_case(seed)
    log(f"seed {seed}: {case.dtype} D={case.head_dim} B={case.block_size} H={case.num_heads} "
        f"Hk={case.num_kv_heads} group={group} "
        f"ctx={case.context_lens.tolist()}")
    g = GpuCase(case)
    kc, vc = case.k_cache, case.v_cache
    for i, (kc, vc) in enumerate(oracle_steps(case)):
        g.run_step(i)
        assert_pool_equal(g.kc, kc, case.dtype, f"seed {seed} K after step {i}")
        assert_pool_equal(g.vc, vc, case.dtype, f"seed {seed} V after step {i}")
    ref = oracle_decode(case, kc, vc)
    out = torch.empty_like(g.q)
    pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=group)
    torch.cuda.synchronize()
    assert_close(out, ref, case.dtype, f"seed {seed} siblings", strict=False)


def random_thin_siblings_case(seed: int) -> tuple:
    """(case, group size) of random thin-grid seed `seed`: one or two long
    prompts (1024 tokens or more) forked into up to 16 samples, so that the
    sibling grid is thin and its tile lists are split (or, where the ids do
    not fit or the ungrouped plan has no workspace, the hint is not taken)."""
    rng = np.random.default_rng([322, 9004, seed])
    dtype = ["f16", "bf16"][seed % 2]
    D = int(rng.choice([64, 128, 256]))
    B = int(rng.choice([8, 16, 32, 64]))
    samples = int(rng.integers(2, 17))
    prompts = int(rng.integers(1, 3))
    prompt_len = int(rng.integers(1024, 3000))
    max_suffix = int(rng.integers(0, 200))
    Hk = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    group = max(2, min(16, samples))
    need = prompts * samples * ((prompt_len + max_suffix) // B + 3)
    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=prompt_len,
                                num_heads=Hk * G, head_dim=D, pool_tokens=max(4096, 2 * need * B), dtype=dtype,
                                max_suffix=max_suffix, num_kv_heads=Hk)
    return case, group


@pytest.mark.parametrize("seed", range(8))
def test_random_thin_siblings(seed):
    case, group = random_thin_siblings_case(seed)
    log(f"thin seed {seed}: {case.dtype} D={case.head_dim} B={case.block_size} H={case.num_heads} "
        f"Hk={case.num_kv_heads} group={group} S={case.q.shape[0]} max_ctx={case.max_context_len}")
    g = GpuCase(case)
    g.run_steps()
    kc, vc = case.k_cache, case.v_cache
    for kc, vc in oracle_steps(case):
        pass
    ref = oracle_decode(case, kc, vc)
    out = torch.empty_like(g.q)
    pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=group)
    torch.cuda.synchronize()
    assert_close(out, ref, case.dtype, f"thin seed {seed} siblings", strict=False)
