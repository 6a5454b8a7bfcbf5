"""pa_swap_blocks on the GPU: preempt (swap out to pinned host memory) and
resume (swap in under new block ids), against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import INT_VIEW, GpuCase, assert_pool_equal, log, pa, to_gpu

pytestmark = pytest.mark.gpu


def pinned_like(a: np.ndarray, dtype: str) -> torch.Tensor:
    """A pinned (page-locked) host tensor holding the bits of ``a``."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).pin_memory().view(torch.bfloat16)
    return torch.from_numpy(a).pin_memory()


def same_bits(t: torch.Tensor, ref: np.ndarray, dtype: str) -> bool:
    """Bitwise equality of a host tensor and a storage array (NaN canaries included)."""
    got = t.view(INT_VIEW[dtype]).numpy()
    return np.array_equal(got, np.ascontiguousarray(ref).view(got.dtype))


def _blocks_of(case, s):
    nb = -(-int(case.context_lens[s]) // case.block_size)
    return [int(b) for b in case.block_tables[s, :nb]]


@pytest.mark.parametrize("dtype,H,D,B", [("f16", 8, 128, 16), ("bf16", 4, 64, 8), ("f32", 2, 32, 4)])
def test_swap_out_and_in_round_trip(dtype, H, D, B):
    case = wl.random_case(51 + D, 5, H, D, B, dtype, ctx_range=(20, 90), spare_blocks=40)
    g = GpuCase(case)
    before = g.decode().clone()
    torch.cuda.synchronize()
    # Preempt sequences 1 and 3: their blocks go to host slots 2, 3, ... (slots 0, 1 stay untouched).
    out_ids = _blocks_of(case, 1) + _blocks_of(case, 3)
    n_host = len(out_ids) + 4
    host_k = wl.canary_fill((n_host,) + case.k_cache.shape[1:], dtype)
    host_v = wl.canary_fill((n_host,) + case.v_cache.shape[1:], dtype)
    hk, hv = pinned_like(host_k, dtype), pinned_like(host_v, dtype)
    out_pairs = np.array([[b, i + 2] for i, b in enumerate(out_ids)], dtype=np.int64)
    log(f"{dtype}: swap out {len(out_ids)} blocks to pinned host memory")
    pa().swap_blocks(hk, hv, g.kc, g.vc, to_gpu(out_pairs))
    torch.cuda.synchronize()
    ref_hk, ref_hv = oracle.swap_blocks(case.k_cache, case.v_cache, host_k, host_v, out_pairs)
    assert same_bits(hk, ref_hk, dtype), "host K after swap-out"
    assert same_bits(hv, ref_hv, dtype), "host V after swap-out"

    # Resume into free device blocks, with the pair list itself in pinned host memory.
    used = {int(b) for b in case.block_tables.ravel() if b >= 0}
    free = [b for b in range(case.num_blocks) if b not in used][: len(out_ids)]
    in_pairs = np.array([[i + 2, f] for i, f in enumerate(free)], dtype=np.int64)
    pairs_h = torch.from_numpy(in_pairs).pin_memory()
    log(f"{dtype}: swap in {len(free)} blocks under new ids")
    pa().swap_blocks(g.kc, g.vc, hk, hv, pairs_h)
    torch.cuda.synchronize()
    ref_kc, ref_vc = oracle.swap_blocks(ref_hk, ref_hv, case.k_cache, case.v_cache, in_pairs)
    assert_pool_equal(g.kc, ref_kc, dtype, "device K after swap-in")
    assert_pool_equal(g.vc, ref_vc, dtype, "device V after swap-in")

    # Decode through the relabelled tables: bit-identical to before the swap.
    bt = case.block_tables.copy()
    n1 = len(_blocks_of(case, 1))
    bt[1, :n1] = free[:n1]
    bt[3, : len(out_ids) - n1] = free[n1:]
    after = g.decode(bt=to_gpu(bt))
    torch.cuda.synchronize()
    iv = INT_VIEW[dtype]
    assert torch.equal(after.view(iv), before.view(iv))


def test_swap_device_to_device_and_skips():
    """Two device pools (a GPU-side swap space); pairs naming ids outside
    either pool are skipped."""
    case = wl.random_case(61, 3, 4, 128, 16, "bf16", ctx_range=(30, 60), spare_blocks=8)
    g = GpuCase(case)
    n_dst = 6
    dst_k = wl.canary_fill((n_dst,) + case.k_cache.shape[1:], "bf16")
    dst_v = wl.canary_fill((n_dst,) + case.v_cache.shape[1:], "bf16")
    dk, dv = to_gpu(dst_k, "bf16"), to_gpu(dst_v, "bf16")
    ids = (_blocks_of(case, 0) + _blocks_of(case, 1) + _blocks_of(case, 2))[:4]
    pairs = np.array([[ids[0], 5], [ids[1], 0], [ids[2], n_dst + 3], [case.num_blocks + 1, 1], [ids[3], 2]],
                     dtype=np.int64)
    pa().swap_blocks(dk, dv, g.kc, g.vc, to_gpu(pairs))
    torch.cuda.synchronize()
    valid = pairs[[0, 1, 4]]
    ref_k, ref_v = oracle.swap_blocks(case.k_cache, case.v_cache, dst_k, dst_v, valid)
    assert_pool_equal(dk, ref_k, "bf16", "device swap space K")
    assert_pool_equal(dv, ref_v, "bf16", "device swap space V")


def test_swap_rejects_pageable_host_memory():
    case = wl.random_case(62, 2, 2, 64, 8, "f16", ctx=[9, 17], spare_blocks=2)
    g = GpuCase(case)
    host = torch.empty((4,) + tuple(case.k_cache.shape[1:]), dtype=torch.float16)  # pageable
    pairs = to_gpu(np.array([[int(case.block_tables[0, 0]), 0]], dtype=np.int64))
    with pytest.raises(ValueError):
        pa().swap_blocks(host, host.clone(), g.kc, g.vc, pairs)
    # Past the binding, the library's own check refuses the pageable pointer
    # before anything is enqueued.  The pair's destination (99) is outside the
    # 4-block pool, so even a launch would skip it and never touch the host
    # memory: a broken check shows as a wrong status, not a fault.
    skip = to_gpu(np.array([[int(case.block_tables[0, 0]), 99]], dtype=np.int64))
    st = pa().lib.pa_swap_blocks(host.data_ptr(), host.data_ptr(), g.kc.data_ptr(), g.vc.data_ptr(),
                                 skip.data_ptr(), 1, 2, 64, 8, case.num_blocks, 4, 1, None)
    torch.cuda.synchronize()
    assert st == 3, pa().status_string(st)
