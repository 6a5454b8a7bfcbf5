"""The relocation the large-pool GPU tests apply (blocks moved to ids
base.., tables, slots and copy pairs shifted), checked on the CPU with the
oracle: the shifted case on a NaN-filled pool computes exactly what the
compact case computes, and nothing below base is touched."""
import numpy as np
import pytest

import oracle
import workloads as wl
from test_gpu_large_pool import shift_slots, shift_tables
from workloads.storage import canary_fill


def relocated_run(case, base):
    shape = (base + case.num_blocks,) + case.k_cache.shape[1:]
    kc, vc = canary_fill(shape, case.dtype), canary_fill(shape, case.dtype)
    kc[base:], vc[base:] = case.k_cache, case.v_cache
    for st in case.steps:
        if isinstance(st, wl.AppendStep):
            kc, vc = oracle.reshape_and_cache(st.key, st.value, kc, vc,
                                              shift_slots(st.slot_mapping, base, case.block_size))
        else:
            kc, vc = oracle.copy_blocks(kc, vc, st.pairs + base)
    out = oracle.paged_decode(case.q, kc, vc, shift_tables(case.block_tables, base), case.context_lens, case.scale,
                              case.dtype)
    return kc, vc, out


@pytest.mark.parametrize("which", ["random", "forked"])
def test_relocated_case_is_the_same_computation(which):
    if which == "random":
        case = wl.random_case(4100, num_seqs=6, num_heads=4, head_dim=16, block_size=8, dtype="f16",
                              ctx_range=(1, 60), n_append=1, num_kv_heads=2)
    else:
        case = wl.parallel_sampling(block_size=8, num_prompts=2, samples=3, prompt_len=30, num_heads=2,
                                    head_dim=16, pool_tokens=512, max_suffix=10)
    base = 7
    kc, vc, out = relocated_run(case, base)
    rk, rv = case.k_cache, case.v_cache
    for st in case.steps:
        if isinstance(st, wl.AppendStep):
            rk, rv = oracle.reshape_and_cache(st.key, st.value, rk, rv, st.slot_mapping)
        else:
            rk, rv = oracle.copy_blocks(rk, rv, st.pairs)
    ref = oracle.paged_decode(case.q, rk, rv, case.block_tables, case.context_lens, case.scale, case.dtype)
    assert np.array_equal(out, ref)
    bits = lambda a: a.view(np.uint16)  # noqa: E731
    assert np.array_equal(bits(kc[base:]), bits(rk)) and np.array_equal(bits(vc[base:]), bits(rv))
    canary = canary_fill((base,) + case.k_cache.shape[1:], case.dtype)
    assert np.array_equal(bits(kc[:base]), bits(canary)) and np.array_equal(bits(vc[:base]), bits(canary))
    # The shift really moves every used block: no shifted id is below base.
    bt = shift_tables(case.block_tables, base)
    assert (bt[case.block_tables >= 0] >= base).all() and (bt[case.block_tables < 0] < 0).all()
