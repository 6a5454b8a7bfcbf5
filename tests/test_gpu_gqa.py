"""Grouped-query attention (num_kv_heads < num_heads) through the C ABI,
against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import GpuCase, assert_close, assert_pool_equal, log, oracle_decode, pa, to_gpu

pytestmark = pytest.mark.gpu


def test_gqa_llama3_8b_shape():
    case = wl.gqa_config("llama3-8b")
    g = GpuCase(case)
    ref = oracle_decode(case, case.k_cache, case.v_cache)
    for part in (0, 256):
        out = g.decode(partition=part, out=torch.empty_like(g.q))
        torch.cuda.synchronize()
        assert_close(out, ref, case.dtype, f"{case.name} partition={part}")


def test_gqa_llama2_70b_tp8_share():
    case = wl.gqa_config("llama2-70b-tp8")
    g = GpuCase(case)
    ref = oracle_decode(case, case.k_cache, case.v_cache)
    for part in (0, 512):
        out = g.decode(partition=part, out=torch.empty_like(g.q))
        torch.cuda.synchronize()
        assert_close(out, ref, case.dtype, f"{case.name} partition={part}")


SWEEP = [
    # dtype, H, Hk, D, B, ctx, partition
    ("f16", 8, 4, 128, 16, [1, 17, 300, 1299], 0),
    ("bf16", 16, 4, 128, 16, [2, 16, 513, 1025], 64),
    ("f32", 8, 1, 64, 8, [5, 100, 901], 100),
    ("f16", 16, 2, 256, 32, [3, 64, 511, 777], 0),
    ("bf16", 8, 1, 128, 16, [1, 4000], 0),
    ("f32", 4, 2, 8, 4, [5, 16, 37], 4),
    ("f16", 32, 4, 64, 1, [1, 2, 129], 16),
    # Default plans of grouped heads: the balanced split (16-bit, D >= 64), or
    # for fp32 / D = 32 its fallback, 256-token partitions on the vector kernel.
    ("f32", 8, 2, 64, 16, [5, 300, 1000], 0),
    ("f16", 8, 2, 32, 8, [3, 260, 513], 0),
    ("bf16", 16, 8, 64, 4, [1, 2, 3, 700, 33, 257], 0),
]


@pytest.mark.parametrize("dtype,H,Hk,D,B,ctx,part", SWEEP,
                         ids=[f"{c[0]}-H{c[1]}-Hk{c[2]}-D{c[3]}-B{c[4]}-P{c[6]}" for c in SWEEP])
def test_gqa_sweep(dtype, H, Hk, D, B, ctx, part):
    case = wl.random_case(500 + H + Hk + D + B, len(ctx), H, D, B, dtype, ctx=ctx, num_kv_heads=Hk, spare_blocks=3)
    g = GpuCase(case)
    ref = oracle_decode(case, case.k_cache, case.v_cache)
    out = g.decode(partition=part, out=torch.empty_like(g.q))
    torch.cuda.synchronize()
    assert_close(out, ref, dtype, f"{case.name} H={H} Hk={Hk}", strict=False)
    # Cached loads: identical bits.
    out2 = g.decode(partition=part, out=torch.empty_like(g.q), shared_blocks=True)
    torch.cuda.synchronize()
    iv = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(out.view(iv), out2.view(iv))


@pytest.mark.parametrize("Hk", [1, 2, 8])
def test_gqa_append_decode(Hk):
    case = wl.random_case(520 + Hk, 5, 8, 128, 16, "f16", ctx=[1, 16, 17, 700, 1500], n_append=1,
                          num_kv_heads=Hk, spare_blocks=3)
    st = case.steps[0]
    assert st.key.shape == (5, Hk, 128)
    g = GpuCase(case)
    out = torch.empty_like(g.q)
    pa().append_decode(out, g.q, to_gpu(st.key, "f16"), to_gpu(st.value, "f16"), g.kc, g.vc, g.bt, g.ctx,
                       case.scale, case.max_context_len)
    torch.cuda.synchronize()
    ref, kc, vc = oracle.append_decode(case.q, st.key, st.value, case.k_cache, case.v_cache, case.block_tables,
                                       case.context_lens, case.scale, "f16")
    assert_pool_equal(g.kc, kc, "f16", f"K Hk={Hk}")
    assert_pool_equal(g.vc, vc, "f16", f"V Hk={Hk}")
    assert_close(out, ref, "f16", f"gqa append_decode Hk={Hk}", strict=False)


def test_balanced_split_empty_invalid_and_tiny_contexts():
    """Balanced split over 200 sequences of 0..40 tokens (many (sequence,
    K/V head) runs per workgroup), one empty context (output 0) and one past
    max_context_len (output NaN, nothing read)."""
    rng = np.random.default_rng(77)
    ctx = rng.integers(1, 41, 200)
    ctx[5] = 0
    case = wl.random_case(540, 200, 8, 128, 16, "f16", ctx=ctx.tolist(), num_kv_heads=2, spare_blocks=3)
    assert pa().partition_tokens(200, 8, case.max_context_len, num_kv_heads=2) == 256  # balanced plan
    g = GpuCase(case)
    bad = case.context_lens.copy()
    bad[7] = case.max_context_len + 1
    out = g.decode(out=torch.full_like(g.q, 7.0), ctx=to_gpu(bad))
    torch.cuda.synchronize()
    seqs = [s for s in range(200) if s not in (5, 7)]
    ref = oracle_decode(case, case.k_cache, case.v_cache, seqs)
    assert_close(out, ref, "f16", "balanced tiny contexts", seqs=seqs)
    o = out.float().cpu()
    assert torch.all(o[5] == 0) and torch.all(torch.isnan(o[7]))
    log("empty context -> 0, invalid context -> NaN")


@pytest.mark.parametrize("H,Hk,D", [(8, 1, 128), (32, 8, 64), (16, 4, 256)])
def test_balanced_split_matches_partitions(H, Hk, D):
    """The balanced split and fixed 256-token partitions both match the
    oracle on a ragged batch with long and short contexts."""
    ctx = [1, 15, 16, 17, 255, 256, 257, 1000, 2500, 40]
    case = wl.random_case(550 + H + D, len(ctx), H, D, 16, "bf16", ctx=ctx, num_kv_heads=Hk, spare_blocks=3)
    g = GpuCase(case)
    ref = oracle_decode(case, case.k_cache, case.v_cache)
    for part in (0, 256):
        out = g.decode(partition=part, out=torch.empty_like(g.q))
        torch.cuda.synchronize()
        assert_close(out, ref, "bf16", f"H={H} Hk={Hk} D={D} partition={part}", strict=False)


@pytest.mark.parametrize("dtype,S,H,Hk", [("f16", 50, 32, 16), ("bf16", 20, 128, 32), ("f16", 70, 32, 8)])
def test_gqa_longest_first_pairing(dtype, S, H, Hk):
    """Grouped-head batches of 512+ (sequence, K/V head) pairs run whole
    contexts longest first, with the second round of grid rows in increasing
    length (paired with the longest in the CUs' first slots): every sequence
    must still be computed exactly once, with its own context.  The batches
    span the paired rows and rows past them."""
    case = wl.random_case(900 + S + Hk, S, H, 128, 16, dtype, ctx_range=(1, 300), num_kv_heads=Hk, spare_blocks=5)
    assert S * Hk >= 512
    g = GpuCase(case)
    ref = oracle_decode(case, case.k_cache, case.v_cache)
    out = g.decode(out=torch.full_like(g.q, float("nan")))
    torch.cuda.synchronize()
    assert_close(out, ref, dtype, f"{case.name} S={S} H={H} Hk={Hk}", strict=False)
