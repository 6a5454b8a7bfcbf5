"""Block pools whose element offsets pass 2^32, against the float64 oracle.

A serving pool on one 288 GB GPU spans tens of gigabytes, so block ids times
the block size overflow 32-bit element offsets.  Each case here is a small
seeded workload whose N blocks are moved to ids base .. base + N - 1 of a
device pool of base + N blocks, with base chosen so that block `base` starts
past element 2^32.  Block tables, slots and copy pairs are shifted by base;
the blocks below base hold NaN canaries, so a truncated offset would read NaN
into the output or write over a canary.  Every kernel is run on such a pool:
append, decode (vector, matrix-core partitioned and balanced plans, sibling
groups), the fused append-decode, copy-on-write copies and prefill.  Outputs
are compared with the oracle run on the compact pool (the oracle's
block-relabelling invariance makes the two the same computation); pools are
compared bit for bit above base and checked untouched below it.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import TORCH_DT, assert_close, assert_pool_equal, log, oracle_steps, pa, to_gpu

pytestmark = pytest.mark.gpu

OFFSET_BITS = 32


def pool_base(case: wl.Case) -> int:
    """First block id whose first element lies past element 2^32."""
    elems = case.num_kv_heads * case.block_size * case.head_dim
    return (1 << OFFSET_BITS) // elems + 1


def shift_tables(bt: np.ndarray, base: int) -> np.ndarray:
    out = bt.copy()
    out[bt >= 0] += base
    return out


def shift_slots(slots: np.ndarray, base: int, block_size: int) -> np.ndarray:
    out = slots.copy()
    out[slots >= 0] += base * block_size
    return out


class BigPool:
    """The case's pool placed at block ids base.. of a NaN-filled device pool."""

    def __init__(self, case: wl.Case):
        self.case, self.base = case, pool_base(case)
        n = self.base + case.num_blocks
        shape = (n, case.num_kv_heads, case.block_size, case.head_dim)
        log(f"{case.name}: pool of {n} blocks, base {self.base} "
            f"({2 * n * np.prod(shape[1:]) * case.elem_bytes / 2**30:.1f} GiB for K and V)")
        assert self.base * np.prod(shape[1:]) > (1 << OFFSET_BITS)
        dt = TORCH_DT[case.dtype]
        self.kc = torch.full(shape, float("nan"), dtype=dt, device="cuda")
        self.vc = torch.full(shape, float("nan"), dtype=dt, device="cuda")
        self.kc[self.base:] = to_gpu(case.k_cache, case.dtype)
        self.vc[self.base:] = to_gpu(case.v_cache, case.dtype)
        self.q = to_gpu(case.q, case.dtype)
        self.bt = to_gpu(shift_tables(case.block_tables, self.base))
        self.ctx = to_gpu(case.context_lens)

    def run_steps(self) -> None:
        c = self.case
        for st in c.steps:
            if isinstance(st, wl.AppendStep):
                pa().reshape_and_cache(to_gpu(st.key, c.dtype), to_gpu(st.value, c.dtype), self.kc, self.vc,
                                       to_gpu(shift_slots(st.slot_mapping, self.base, c.block_size)))
            else:
                pa().copy_blocks(self.kc, self.vc, to_gpu(st.pairs + self.base))

    def check_pools(self, kc: np.ndarray, vc: np.ndarray, what: str) -> None:
        torch.cuda.synchronize()
        assert_pool_equal(self.kc[self.base:], kc, self.case.dtype, f"{what} K above base")
        assert_pool_equal(self.vc[self.base:], vc, self.case.dtype, f"{what} V above base")
        assert bool(torch.isnan(self.kc[:self.base]).all()), f"{what}: K written below base"
        assert bool(torch.isnan(self.vc[:self.base]).all()), f"{what}: V written below base"

    def free(self) -> None:
        del self.kc, self.vc
        torch.cuda.empty_cache()


def final_pools(case):
    kc, vc = case.k_cache, case.v_cache
    for kc, vc in oracle_steps(case):
        pass
    return kc, vc


def decode_vs_oracle(case, partitions=(0,), siblings=0):
    big = BigPool(case)
    try:
        big.run_steps()
        kc, vc = final_pools(case)
        big.check_pools(kc, vc, case.name)
        ref = oracle.paged_decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
        for p in partitions:
            out = torch.empty_like(big.q)
            log(f"{case.name}: decode partition={p} siblings={siblings}")
            pa().decode(out, big.q, big.kc, big.vc, big.bt, big.ctx, case.scale, case.max_context_len,
                        partition_size=p, siblings=siblings)
            torch.cuda.synchronize()
            assert_close(out, ref, case.dtype, f"{case.name} large pool partition={p} siblings={siblings}")
    finally:
        big.free()


DECODE_CASES = [
    # name, dtype, H, Hk, D, B, ctx range, partitions
    ("vector-f16", "f16", 8, 8, 128, 16, (1, 700), (0, 64)),
    ("vector-f32", "f32", 4, 4, 64, 8, (1, 300), (0, 40)),
    ("mfma-bf16-g4", "bf16", 16, 4, 128, 16, (1, 900), (0, 128)),
    ("mfma-f16-g8", "f16", 8, 1, 128, 32, (1, 1500), (0,)),
]


@pytest.mark.parametrize("name,dtype,H,Hk,D,B,rng,parts", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_large_pool_append_then_decode(name, dtype, H, Hk, D, B, rng, parts):
    case = wl.random_case(4100 + len(name), num_seqs=12, num_heads=H, head_dim=D, block_size=B, dtype=dtype,
                          ctx_range=rng, n_append=1, num_kv_heads=Hk)
    decode_vs_oracle(case, partitions=parts)


def test_large_pool_forked_samples():
    # Copy-on-write fork copies at high block ids, then decode one sequence
    # at a time and in sibling groups.
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=4, prompt_len=200, num_heads=8,
                                head_dim=128, pool_tokens=8192, max_suffix=40)
    assert any(isinstance(st, wl.CopyStep) for st in case.steps)
    decode_vs_oracle(case, partitions=(0,), siblings=0)
    decode_vs_oracle(case, partitions=(0,), siblings=4)


def test_large_pool_append_decode():
    case = wl.random_case(4200, num_seqs=12, num_heads=8, head_dim=128, block_size=16, dtype="f16",
                          ctx_range=(1, 700), n_append=1)
    st = case.steps[0]
    assert st.slot_mapping.size == case.num_seqs
    big = BigPool(case)
    try:
        out = torch.empty_like(big.q)
        log(f"{case.name}: append_decode on the large pool")
        pa().append_decode(out, big.q, to_gpu(st.key, case.dtype), to_gpu(st.value, case.dtype), big.kc, big.vc,
                           big.bt, big.ctx, case.scale, case.max_context_len)
        kc, vc = final_pools(case)
        big.check_pools(kc, vc, f"{case.name} append_decode")
        ref = oracle.paged_decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
        assert_close(out, ref, case.dtype, f"{case.name} large pool append_decode")
    finally:
        big.free()


@pytest.mark.parametrize("dtype,H,Hk,D", [("f16", 8, 8, 128), ("bf16", 8, 2, 64)])
def test_large_pool_prefill(dtype, H, Hk, D):
    case = wl.random_prefill_case(4300 + D, prefix=[0, 37, 300, 1000], chunk=[130, 1, 64, 200], num_heads=H,
                                  head_dim=D, block_size=16, dtype=dtype, num_kv_heads=Hk)
    big = BigPool(case)
    try:
        big.run_steps()
        kc, vc = final_pools(case)
        big.check_pools(kc, vc, case.name)
        out = torch.full_like(big.q, float("nan"))
        qs = to_gpu(case.query_start)
        mq = int(np.diff(case.query_start).max())
        log(f"{case.name}: prefill on the large pool")
        pa().prefill(out, big.q, big.kc, big.vc, big.bt, big.ctx, qs, case.scale, mq, case.max_context_len)
        torch.cuda.synchronize()
        ref = oracle.paged_prefill(case.q, kc, vc, case.block_tables, case.context_lens, case.query_start,
                                   case.scale, case.dtype)
        assert_close(out, ref, case.dtype, f"{case.name} large pool prefill", strict=dtype == "f16")
    finally:
        big.free()
