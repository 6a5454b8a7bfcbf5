"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: max-abs 2e-3 for f16/bf16 inputs and 1e-5 for f32 inputs on the
attention output; cache writes and block copies bit-exact over the whole
pool (compared as integers, so NaN canaries compare too).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import GpuCase, assert_close, assert_pool_equal, log, oracle_decode, oracle_steps, pa

pytestmark = pytest.mark.gpu


def full_parity(case: wl.Case, partitions=(0,), seqs=None, strict=True):
    g = GpuCase(case)
    kc, vc = case.k_cache, case.v_cache
    for i, (kc, vc) in enumerate(oracle_steps(case)):
        log(f"{case.name}: step {i}")
        g.run_step(i)
        assert_pool_equal(g.kc, kc, case.dtype, f"{case.name} K after step {i}")
        assert_pool_equal(g.vc, vc, case.dtype, f"{case.name} V after step {i}")
    ref = oracle_decode(case, kc, vc, seqs)
    for p in partitions:
        log(f"{case.name}: decode partition={p}")
        out = g.decode(partition=p)
        torch.cuda.synchronize()
        assert_close(out, ref, case.dtype, f"{case.name} partition={p}", seqs=seqs, strict=strict)
    return g, ref


def test_tiny_f32():
    full_parity(wl.tiny_f32(), partitions=(0, 4, 8, 12, 37))


def test_llama7b_decode_shape():
    full_parity(wl.llama7b_decode(), partitions=(0, 256))


def test_opt13b_append_then_decode():
    full_parity(wl.opt13b_decode())


@pytest.mark.parametrize("B", [8, 16, 32])
def test_parallel_sampling_cow(B):
    g, ref = full_parity(wl.parallel_sampling(block_size=B))
    # Cached loads for shared blocks: a cache policy only, results bit-identical.
    streamed = g.decode(out=torch.empty_like(g.q)).clone()
    cached = g.decode(out=torch.empty_like(g.q), shared_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(cached.view(torch.int16), streamed.view(torch.int16))


def test_opt175b_shape():
    # Every sequence of the OPT-175B-shaped batch, at the default plan (whole
    # contexts) and with contexts split into 512-token partitions, so the
    # split-K merge runs at this shape too.
    full_parity(wl.opt175b_decode(), partitions=(0, 512))


@pytest.mark.parametrize("kind", ["mha", "gqa"])
def test_wide_batch_of_short_contexts(kind):
    """12000 sequences of 0-96 tokens (some empty): tens of thousands of
    workgroups in batch order, every sequence against the oracle, at the
    default plan and split into 32-token partitions (the merge over 24000 or
    96000 (sequence, head) rows); for the grouped-query batch also as
    sibling groups of 4 unrelated sequences (nothing shared)."""
    if kind == "mha":
        case = wl.random_case(92, 12000, 2, 64, 16, "f16", ctx_range=(0, 96))
    else:
        case = wl.random_case(91, 12000, 8, 64, 16, "bf16", ctx_range=(0, 96), num_kv_heads=2)
    # bf16 rows that see a few keys reach |out| ~ 3, where one output ulp exceeds 2e-3.
    g, ref = full_parity(case, partitions=(0, 32), strict=case.dtype == "f16")
    if kind == "gqa":
        out = torch.full_like(g.q, float("nan"))
        pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=4)
        torch.cuda.synchronize()
        assert_close(out, ref, case.dtype, f"{case.name} siblings=4", strict=False)


@pytest.mark.parametrize("kind", ["mha", "gqa"])
def test_128k_token_contexts(kind):
    """Contexts of 131072, 70001, 1 and 0 tokens.  The default plan cuts the
    longest into 512 partitions of 256 tokens (multi-head: more than the
    merge kernel's 256 cached weights) or, for one K/V head of 8 query heads,
    into a balanced split of a few hundred pieces; also 4096-token
    partitions."""
    if kind == "mha":
        case = wl.random_case(93, 4, 4, 128, 16, "f16", ctx=[131072, 70001, 1, 0])
    else:
        case = wl.random_case(94, 4, 8, 128, 16, "bf16", ctx=[131072, 70001, 1, 0], num_kv_heads=1)
    full_parity(case, partitions=(0, 4096))


def test_opt175b_tp8_share():
    # One tensor-parallel rank's share of the OPT-175B-shaped layer: 96 heads
    # over 8 GPUs leave 12 per GPU, with the same block tables and lengths.
    full_parity(wl.opt175b_decode(num_heads=12), partitions=(0, 512))


SWEEP = [
    # dtype, head_dim, block_size, ctx, partition
    ("f32", 128, 16, [1, 17, 300, 1299], 0),
    ("f16", 128, 16, [1, 15, 16, 17, 513, 1300], 64),
    ("bf16", 128, 32, [2, 33, 700, 1025], 0),
    ("f16", 64, 8, [5, 100, 900], 100),
    ("bf16", 256, 16, [3, 64, 511, 512, 777], 128),
    ("f32", 256, 4, [7, 260], 32),
    ("f16", 8, 1, [1, 2, 3, 64, 129], 16),
    ("f32", 8, 4, [5, 16, 37], 0),
    ("f16", 16, 2, [9, 40], 8),
    ("bf16", 32, 64, [65, 200], 0),
    ("f16", 128, 256, [1, 257, 600], 0),
]


@pytest.mark.parametrize("dtype,D,B,ctx,part", SWEEP, ids=[f"{s[0]}-D{s[1]}-B{s[2]}-P{s[4]}" for s in SWEEP])
def test_shape_sweep(dtype, D, B, ctx, part):
    case = wl.random_case(100 + D + B, len(ctx), 3, D, B, dtype, ctx=ctx, spare_blocks=7)
    # Short contexts give |out| near 1-3, where f16/bf16 rounding alone
    # exceeds 2e-3: the bound here is 2e-3 or one output ulp.
    full_parity(case, partitions=(part,), strict=False)


@pytest.mark.parametrize("dtype,G", [("f32", 1), ("f16", 1), ("bf16", 1), ("f16", 4), ("bf16", 8)])
@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_zero_and_negative_scale(dtype, G, scale):
    """Scale 0 gives the plain mean of each context's V rows (tail slots of
    the last block, NaN-poisoned, must weigh exactly 0); a negative scale is
    an ordinary softmax of the negated scores.  Both decode kernels (vector
    for G = 1, matrix-core for grouped heads) and a forced split."""
    case = wl.random_case(77 + G, 4, 2 * G, 128, 16, dtype, ctx=[1, 15, 100, 700], spare_blocks=5, scale=scale,
                          num_kv_heads=2)
    full_parity(case, partitions=(0, 64), strict=False)


def test_append_sweep():
    for dtype, D, B in (("f32", 64, 4), ("bf16", 128, 16), ("f16", 256, 32)):
        case = wl.random_case(200 + D, 5, 4, D, B, dtype, ctx_range=(3, 90), n_append=3, spare_blocks=6)
        st = case.steps[0]
        # An extra padding row (slot -1) that belongs to no sequence is skipped.
        pad = np.zeros((1,) + st.key.shape[1:], dtype=st.key.dtype)
        st.key = np.concatenate([st.key[:2], pad, st.key[2:]])
        st.value = np.concatenate([st.value[:2], pad, st.value[2:]])
        st.slot_mapping = np.concatenate([st.slot_mapping[:2], [-1], st.slot_mapping[2:]]).astype(np.int64)
        full_parity(case, strict=False)


def test_context_len_zero_and_one():
    for dtype in wl.DTYPES:
        case = wl.random_case(300, 4, 2, 128, 16, dtype, ctx=[0, 1, 1, 0])
        g = GpuCase(case)
        out = g.decode()
        torch.cuda.synchronize()
        got = out.double().cpu().numpy()
        assert (got[0] == 0).all() and (got[3] == 0).all()
        for s in (1, 2):
            b = case.block_tables[s, 0]
            v = g.vc[b, :, 0, :]
            assert torch.equal(out[s].view(torch.int16 if dtype != "f32" else torch.int32),
                               v.view(torch.int16 if dtype != "f32" else torch.int32)), dtype


def test_longest_context_and_full_table():
    # A context that uses every entry of its table row, 8192 tokens long.
    case = wl.random_case(301, 2, 2, 128, 16, "f16", ctx=[8192, 4097], spare_blocks=2)
    assert case.block_tables.shape[1] * 16 == 8192
    full_parity(case, partitions=(0, 2048))


def test_16bit_partition_beyond_matrix_core_staging():
    # 16-bit caches normally take the matrix-core kernel; a partition that
    # stages more than 6144 block ids (block size 1, 6300-token partition)
    # takes the vector kernel instead.  Both must agree with the oracle.
    case = wl.random_case(303, 2, 4, 128, 1, "bf16", ctx=[6400, 700], spare_blocks=3, num_kv_heads=1)
    full_parity(case, partitions=(6300, 0), strict=False)


def test_head_dim_256_staging_limit():
    # At head_dim 256 the matrix-core kernel's per-wavefront tiles take
    # 143 KB of LDS, so it stages at most 4096 block ids: a 4000-token
    # partition of 1-token blocks runs on the matrix cores (159 KB of LDS in
    # all), a 5000-token one on the vector kernel; both match the oracle, as
    # does the default plan (a balanced split).
    case = wl.random_case(304, 2, 8, 256, 1, "f16", ctx=[5200, 300], spare_blocks=3, num_kv_heads=2)
    full_parity(case, partitions=(4000, 5000, 0), strict=False)


def test_empty_calls_are_no_ops():
    case = wl.random_case(302, 2, 2, 64, 8, "f16", ctx=[3, 9])
    g = GpuCase(case)
    before_k = g.kc.clone()
    e16 = torch.empty(0, 2, 64, dtype=torch.float16, device="cuda")
    pa().reshape_and_cache(e16, e16, g.kc, g.vc, torch.empty(0, dtype=torch.int64, device="cuda"))
    pa().copy_blocks(g.kc, g.vc, torch.empty(0, 2, dtype=torch.int64, device="cuda"))
    out0 = torch.empty(0, 2, 64, dtype=torch.float16, device="cuda")
    pa().decode(out0, out0, g.kc, g.vc, g.bt[:0], g.ctx[:0], 0.1, 0)
    torch.cuda.synchronize()
    assert torch.equal(before_k.view(torch.int16), g.kc.view(torch.int16))


def test_block_relabelling_is_bitwise_invariant():
    case = wl.random_case(303, 6, 4, 128, 16, "bf16", ctx_range=(1, 1500), spare_blocks=11)
    g = GpuCase(case)
    base = g.decode().clone()
    pi = torch.from_numpy(np.random.default_rng(5).permutation(case.num_blocks)).cuda()
    kc = torch.empty_like(g.kc)
    vc = torch.empty_like(g.vc)
    kc[pi] = g.kc
    vc[pi] = g.vc
    bt = torch.where(g.bt >= 0, pi[g.bt.clamp(min=0).long()].int(), g.bt)
    out = g.decode(out=torch.empty_like(base), bt=bt, kc=kc, vc=vc)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_split_partitions_agree():
    """Any KV partition size gives the same result up to fp32 summation order:
    outputs are O(1) (convex combinations of N(0,1) rows), so the bound is
    absolute, 1e-6, and every split also matches the oracle to 1e-5."""
    case = wl.random_case(304, 5, 4, 128, 16, "f32", ctx=[2048, 1999, 1024, 513, 64])
    g = GpuCase(case)
    outs = {p: g.decode(partition=p, out=torch.empty_like(g.q)) for p in (16, 64, 100, 512, 2048)}
    torch.cuda.synchronize()
    ref = outs[2048].double()
    oref = oracle_decode(case, case.k_cache, case.v_cache)
    for p, o in outs.items():
        d = (o.double() - ref).abs().max().item()
        log(f"split {p} vs unsplit: max abs diff {d:.2e}")
        assert d <= 1e-6, p
        assert_close(o, oref, "f32", f"split {p}")


def test_fork_reads_through_copy_bitwise():
    case = wl.parallel_sampling(block_size=16, num_prompts=4, num_heads=8, head_dim=128, pool_tokens=16384)
    g = GpuCase(case)
    g.run_step(0)
    g.run_step(1)
    pre_ctx = torch.full_like(g.ctx, 500)
    forked = g.decode(ctx=pre_ctx, max_context_len=500, out=torch.empty_like(g.q)).clone()
    bt = g.bt.clone()
    for p in range(4):
        bt[4 * p : 4 * p + 4] = g.bt[4 * p + 3]  # every sample reads the original blocks
    shared = g.decode(ctx=pre_ctx, bt=bt, max_context_len=500, out=torch.empty_like(g.q))
    torch.cuda.synchronize()
    assert torch.equal(forked.view(torch.int16), shared.view(torch.int16))


def test_out_of_pool_block_id_gives_nan():
    case = wl.random_case(305, 3, 2, 64, 8, "f16", ctx=[20, 20, 5])
    g = GpuCase(case)
    bt = g.bt.clone()
    bt[0, 1] = case.num_blocks + 100  # outside the pool: the kernel must not read it
    bt[2, 0] = -3
    out = g.decode(bt=bt)
    torch.cuda.synchronize()
    got = out.float().cpu()
    assert torch.isnan(got[0]).all() and torch.isnan(got[2]).all()
    assert torch.isfinite(got[1]).all()


def test_runs_on_a_side_stream():
    case = wl.random_case(306, 4, 4, 128, 16, "f16", ctx_range=(100, 900))
    g = GpuCase(case)
    ref = g.decode(out=torch.empty_like(g.q)).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = g.decode(out=torch.empty_like(g.q), partition=128)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert (out.float() - ref.float()).abs().max().item() <= 2e-3


def test_workspace_reusable_across_shapes():
    """One workspace buffer (never cleared) serves any sequence of calls, of
    any shape: its contents need no initialisation."""
    ws = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
    cases = [
        wl.random_case(307, 5, 4, 128, 16, "f16", ctx=[700, 33, 1500, 16, 1025], spare_blocks=3),
        wl.random_case(308, 9, 2, 64, 8, "bf16", ctx_range=(1, 900), spare_blocks=5),
        wl.random_case(309, 3, 8, 256, 32, "f32", ctx=[4000, 100, 2049], spare_blocks=2),
    ]
    for rep in range(2):
        for case in cases:
            g = GpuCase(case)
            ref = oracle_decode(case, case.k_cache, case.v_cache)
            for part in (16, 96, 512):
                need = pa().decode_workspace_size(case.num_seqs, case.num_heads, case.head_dim,
                                                  case.max_context_len, part)
                assert 0 < need <= ws.numel()
                out = torch.empty_like(g.q)
                pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len,
                            partition_size=part, workspace=ws)
                torch.cuda.synchronize()
                assert_close(out, ref, case.dtype, f"{case.name} part={part} rep={rep}", strict=False)


def test_split_merge_is_deterministic():
    """The merge sums partitions in a fixed order: repeated calls agree bitwise."""
    case = wl.random_case(310, 16, 8, 128, 16, "f16", ctx_range=(1000, 2048), spare_blocks=4)
    g = GpuCase(case)
    first = g.decode(partition=64, out=torch.empty_like(g.q)).clone()
    for _ in range(5):
        again = g.decode(partition=64, out=torch.empty_like(g.q))
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))


def test_many_sequences_batch_order():
    """More than 512 sequences: contexts are split and dispatched in batch order."""
    case = wl.random_case(311, 600, 1, 64, 8, "f16", ctx_range=(1, 700), spare_blocks=9)
    assert pa().partition_tokens(600, 1, case.max_context_len) == 256
    full_parity(case, partitions=(0,), strict=False)


def test_longest_first_order_whole_contexts():
    """1024..8191 (sequence, head) pairs over <= 512 sequences: whole contexts,
    longest first (the LLaMA-7B-shaped batch takes this path)."""
    case = wl.random_case(312, 40, 32, 128, 16, "bf16", ctx_range=(1, 1500), spare_blocks=5)
    assert pa().partition_tokens(40, 32, case.max_context_len) >= case.max_context_len
    assert pa().decode_workspace_size(40, 32, 128, case.max_context_len) == 0
    full_parity(case, partitions=(0,), strict=False)  # short contexts: bf16 rounding can exceed 2e-3
