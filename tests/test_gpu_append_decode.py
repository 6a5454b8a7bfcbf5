"""pa_append_decode (store each sequence's newest K/V row, then attend, in one
launch) against the oracle and against pa_reshape_and_cache + pa_decode
(bit-identical caches and outputs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import GpuCase, assert_close, assert_pool_equal, log, pa, to_gpu

pytestmark = pytest.mark.gpu


def fused_vs_oracle(case, seqs=None, partition=0, strict=True):
    st = case.steps[0]
    assert st.slot_mapping.size == case.num_seqs
    g = GpuCase(case)
    k_new, v_new = to_gpu(st.key, case.dtype), to_gpu(st.value, case.dtype)
    out = torch.empty_like(g.q)
    log(f"{case.name}: append_decode partition={partition}")
    pa().append_decode(out, g.q, k_new, v_new, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len,
                       partition_size=partition)
    torch.cuda.synchronize()
    slots = oracle.newest_token_slots(case.block_tables, case.context_lens, case.block_size)
    assert np.array_equal(slots, st.slot_mapping)
    kc, vc = oracle.reshape_and_cache(st.key, st.value, case.k_cache, case.v_cache, slots)
    assert_pool_equal(g.kc, kc, case.dtype, f"{case.name} K after append_decode")
    assert_pool_equal(g.vc, vc, case.dtype, f"{case.name} V after append_decode")
    idx = np.arange(case.num_seqs) if seqs is None else np.asarray(seqs)
    ref = oracle.paged_decode(case.q[idx], kc, vc, case.block_tables[idx], case.context_lens[idx], case.scale,
                              case.dtype)
    assert_close(out, ref, case.dtype, f"{case.name} append_decode", seqs=seqs, strict=strict)


def test_append_decode_llama7b_shape():
    fused_vs_oracle(wl.llama7b_decode(n_append=1))


def test_append_decode_opt13b_shape():
    fused_vs_oracle(wl.opt13b_decode())


def test_append_decode_opt175b_shape():
    fused_vs_oracle(wl.opt175b_decode(n_append=1))


def test_append_decode_opt175b_shape_split():
    fused_vs_oracle(wl.opt175b_decode(n_append=1), partition=512)


CASES = [
    # dtype, D, B, ctx, partition
    ("f16", 128, 16, [1, 16, 17, 33, 500, 1025], 0),
    ("f16", 128, 16, [1, 16, 17, 33, 500, 1025], 16),
    ("bf16", 64, 8, [2, 9, 257, 300], 100),
    ("f32", 8, 4, [5, 16, 37], 4),
    ("f32", 256, 32, [1, 64, 65, 700], 0),
]


@pytest.mark.parametrize("dtype,D,B,ctx,part", CASES, ids=[f"{c[0]}-D{c[1]}-B{c[2]}-P{c[4]}" for c in CASES])
def test_append_decode_equals_two_calls(dtype, D, B, ctx, part):
    case = wl.random_case(400 + D + B + part, len(ctx), 3, D, B, dtype, ctx=ctx, n_append=1, spare_blocks=4)
    fused_vs_oracle(case, partition=part, strict=False)
    st = case.steps[0]
    a, b = GpuCase(case), GpuCase(case)
    out_a, out_b = torch.empty_like(a.q), torch.empty_like(b.q)
    pa().append_decode(out_a, a.q, to_gpu(st.key, dtype), to_gpu(st.value, dtype), a.kc, a.vc, a.bt, a.ctx,
                       case.scale, case.max_context_len, partition_size=part)
    pa().reshape_and_cache(to_gpu(st.key, dtype), to_gpu(st.value, dtype), b.kc, b.vc, to_gpu(st.slot_mapping))
    b.decode(partition=part, out=out_b)
    torch.cuda.synchronize()
    iv = torch.int32 if dtype == "f32" else torch.int16
    # The fused kernel reads the newest token in the same slot of the same
    # step as the two-launch path: caches and output are bit-identical.
    assert torch.equal(a.kc.view(iv), b.kc.view(iv)) and torch.equal(a.vc.view(iv), b.vc.view(iv))
    assert torch.equal(out_a.view(iv), out_b.view(iv))


def test_append_decode_empty_context_stores_nothing():
    case = wl.random_case(420, 3, 2, 64, 8, "f16", ctx=[0, 9, 0], spare_blocks=2)
    g = GpuCase(case)
    rng = np.random.default_rng(1)
    key = wl.to_storage(rng.standard_normal((3, 2, 64), dtype=np.float32), "f16")
    value = wl.to_storage(rng.standard_normal((3, 2, 64), dtype=np.float32), "f16")
    out = torch.empty_like(g.q)
    pa().append_decode(out, g.q, to_gpu(key), to_gpu(value), g.kc, g.vc, g.bt, g.ctx, case.scale,
                       case.max_context_len)
    torch.cuda.synchronize()
    ref, kc, vc = oracle.append_decode(case.q, key, value, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.scale, "f16")
    assert_pool_equal(g.kc, kc, "f16", "K")
    assert_pool_equal(g.vc, vc, "f16", "V")
    assert_close(out, ref, "f16", "append_decode with empty contexts", strict=False)
    assert (out[0].float() == 0).all() and (out[2].float() == 0).all()
