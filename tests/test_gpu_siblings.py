"""Sibling-group decode (pa_decode with PA_DECODE_SIBLINGS(n)): the shared
leading blocks of forked samples read once per group, against the oracle on
every sequence, and against the ungrouped decode (same definition; the two
differ by fp32 rounding only).  Multi-head and grouped-query heads,
groups cut into sub-groups where members x query heads exceed the 16
matrix columns, unrelated sequences, empty, impossible and out-of-pool
entries, and the cases where the hint is not taken."""
import pytest
import torch

import workloads as wl
from gpu_helpers import GpuCase, assert_close, log, oracle_decode, oracle_steps, pa

pytestmark = pytest.mark.gpu


def run_case(case, group, strict=True, shared_blocks=False):
    g = GpuCase(case)
    g.run_steps()
    kc, vc = case.k_cache, case.v_cache
    for kc, vc in oracle_steps(case):
        pass
    ref = oracle_decode(case, kc, vc)
    out = torch.full_like(g.q, float("nan"))
    pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, shared_blocks=shared_blocks,
                siblings=group)
    plain = g.decode(out=torch.empty_like(g.q), shared_blocks=shared_blocks)
    torch.cuda.synchronize()
    assert_close(out, ref, case.dtype, f"{case.name} siblings={group}", strict=strict)
    diff = (out.float() - plain.float()).abs().max().item()
    log(f"{case.name}: max |grouped - ungrouped| = {diff:.3e}")
    return g, out, ref


@pytest.mark.parametrize("B", [8, 16, 32])
def test_parallel_sampling_siblings(B):
    # 64 prompts x 4 samples: prompt blocks shared, the partly filled last
    # prompt block copied for samples 0-2 at the fork.
    case = wl.parallel_sampling(block_size=B)
    g, out, ref = run_case(case, 4)
    # Cached instead of streaming loads: a cache policy only, identical bits.
    cached = torch.empty_like(g.q)
    pa().decode(cached, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, shared_blocks=True,
                siblings=4)
    torch.cuda.synchronize()
    assert torch.equal(cached.view(torch.int16), out.view(torch.int16))


SIB_CASES = [
    # seed, group, dtype, D, B, prompts, samples, prompt_len, max_suffix
    (1, 2, "f16", 64, 1, 3, 2, 37, 20),
    (2, 3, "bf16", 128, 8, 4, 3, 100, 40),
    (3, 16, "f16", 128, 16, 2, 16, 70, 30),
    (4, 4, "bf16", 256, 32, 3, 4, 65, 64),
    (5, 5, "f16", 128, 256, 3, 4, 300, 10),  # groups cut across prompts
]


@pytest.mark.parametrize("seed,group,dtype,D,B,prompts,samples,plen,msuf", SIB_CASES,
                         ids=[f"n{c[1]}-{c[2]}-D{c[3]}-B{c[4]}" for c in SIB_CASES])
def test_siblings_forked(seed, group, dtype, D, B, prompts, samples, plen, msuf):
    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=plen, num_heads=2,
                                head_dim=D, pool_tokens=max(4096, 64 * B), dtype=dtype, max_suffix=msuf)
    # Short contexts give |out| near 1-3: 2e-3 or one output ulp.
    run_case(case, group, strict=False)


def test_siblings_unrelated_sequences_and_guards():
    """Sequences that share nothing (every token read privately), an empty
    context (zeros), an impossible context (NaN for that member only) and an
    out-of-pool id in one member's own blocks (NaN for that member only)."""
    case = wl.random_case(77, 7, 2, 128, 16, "f16", ctx=[1, 300, 0, 17, 64, 65, 900], spare_blocks=4)
    g, out, ref = run_case(case, 4, strict=False)
    assert (out[2].float() == 0).all()
    run_case(case, 3, strict=False)
    # Impossible context for sequence 1 (group 0 of 4): NaN there only.
    ctx = case.context_lens.copy()
    ctx[1] = case.max_context_len + 5
    out = torch.full_like(g.q, 0.0)
    pa().decode(out, g.q, g.kc, g.vc, g.bt, torch.from_numpy(ctx).cuda(), case.scale, case.max_context_len,
                siblings=4)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all()
    keep = [0, 2, 3, 4, 5, 6]
    assert_close(out[keep], ref[keep], "f16", "siblings: other members", strict=False)
    # Out-of-pool id in sequence 6's last block.
    bt = case.block_tables.copy()
    bt[6, (int(case.context_lens[6]) - 1) // case.block_size] = case.num_blocks + 3
    out = torch.full_like(g.q, 0.0)
    pa().decode(out, g.q, g.kc, g.vc, torch.from_numpy(bt).cuda(), g.ctx, case.scale, case.max_context_len,
                siblings=4)
    torch.cuda.synchronize()
    assert torch.isnan(out[6].float()).all()
    keep = [0, 1, 2, 3, 4, 5]
    assert_close(out[keep], ref[keep], "f16", "siblings: bad id elsewhere", strict=False)


def test_siblings_bad_id_in_the_shared_prefix():
    """An out-of-pool id in the blocks a whole group shares gives NaN for
    every member of that group and nothing else."""
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=4, prompt_len=100, num_heads=2, head_dim=128,
                                pool_tokens=8192, max_suffix=30)
    g, out, ref = run_case(case, 4, strict=False)
    bt = case.block_tables.copy()
    bt[4:8, 1] = case.num_blocks + 1  # group 1, a shared prompt block
    out = torch.full_like(g.q, 0.0)
    pa().decode(out, g.q, g.kc, g.vc, torch.from_numpy(bt).cuda(), g.ctx, case.scale, case.max_context_len,
                siblings=4)
    torch.cuda.synchronize()
    assert torch.isnan(out[4:8].float()).all()
    keep = [0, 1, 2, 3, 8, 9, 10, 11]
    assert_close(out[keep], ref[keep], "f16", "siblings: other groups", strict=False)


@pytest.mark.parametrize("G,group,dtype", [(2, 4, "f16"), (4, 4, "bf16"), (8, 2, "f16"), (4, 3, "f16")])
def test_siblings_grouped_query(G, group, dtype):
    """Grouped-query heads: member m of a group takes matrix columns
    m G .. m G + G - 1 (n G <= 16); each K/V tile of the shared prefix feeds
    every member's G query heads at once."""
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=4, prompt_len=90, num_heads=2 * G,
                                head_dim=128, pool_tokens=8192, max_suffix=40, num_kv_heads=2, dtype=dtype)
    run_case(case, group, strict=False)


def test_siblings_grouped_query_llama3_8b_shape():
    """LLaMA-3-8B-shaped heads (32 query over 8 K/V heads) for 16 prompts x 4
    samples: 4 members x 4 query heads fill the 16 columns."""
    case = wl.parallel_sampling(block_size=16, num_prompts=16, samples=4, prompt_len=500, num_heads=32,
                                head_dim=128, pool_tokens=65536, num_kv_heads=8)
    run_case(case, 4)


@pytest.mark.parametrize("G,group,dtype,D", [(8, 4, "f16", 128), (8, 3, "bf16", 128), (4, 8, "f16", 128),
                                             (2, 16, "bf16", 128), (8, 16, "f16", 128), (8, 4, "bf16", 256),
                                             (4, 6, "f16", 64)])
def test_siblings_subgroups(G, group, dtype, D):
    """Members x query heads above the 16 matrix columns: each group is cut
    into consecutive sub-groups of min(n, 16 // G) members, one workgroup
    each (a group's last sub-group may be smaller, down to one member)."""
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=max(group, 4), prompt_len=90,
                                num_heads=2 * G, head_dim=D, pool_tokens=16384, max_suffix=40, num_kv_heads=2,
                                dtype=dtype)
    g, out, ref = run_case(case, group, strict=False)
    sub = 16 // G
    if group % sub == 0:
        # Sub-groups of an aligned larger group are the groups of size
        # `sub`: the same workgroups, the same bits.
        small = torch.empty_like(g.q)
        pa().decode(small, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=sub)
        torch.cuda.synchronize()
        assert torch.equal(small.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("what", ["f32", "ids", "d32"])
def test_siblings_hint_ignored_where_not_built(what):
    """Where the sibling kernel is not built or the members' block ids do
    not fit its LDS (fp32 caches, more than 4096 ids per workgroup, head_dim
    below 64) the hint changes nothing: identical bits."""
    group = 3
    if what == "f32":
        case = wl.random_case(81, 6, 2, 64, 8, "f32", ctx=[5, 40, 41, 9, 100, 3], spare_blocks=2)
    elif what == "ids":
        # B = 1: 3 members x 2100 ids > 4096.
        case = wl.random_case(82, 6, 2, 64, 1, "f16", ctx=[5, 40, 41, 9, 2100, 3], spare_blocks=2)
    else:
        case = wl.random_case(83, 6, 2, 32, 16, "bf16", ctx=[5, 40, 41, 9, 100, 3], spare_blocks=2)
    g = GpuCase(case)
    a = g.decode(out=torch.empty_like(g.q)).clone()
    b = torch.empty_like(g.q)
    pa().decode(b, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=group)
    torch.cuda.synchronize()
    iv = torch.int32 if case.dtype == "f32" else torch.int16
    assert torch.equal(a.view(iv), b.view(iv))


def _thin_case(Hk, prompts=1):
    # One (or two) 1200-token prompts forked into 16 samples each: a single
    # round of one workgroup per (sub-group, K/V head) would be 32 or 64
    # workgroups for the whole GPU.
    return wl.parallel_sampling(block_size=16, num_prompts=prompts, samples=16, prompt_len=1200, num_heads=32,
                                head_dim=128, pool_tokens=32768, max_suffix=64, num_kv_heads=Hk)


@pytest.mark.parametrize("Hk", [8, 32])
def test_siblings_thin_grid_split(Hk):
    """A thin grid over long contexts splits each tile list over several
    workgroups (their partials merged as split contexts are): the oracle's
    values, every member, and the same bits from pa_decode_static (the
    same kernels with the library's scratch as workspace)."""
    case = _thin_case(Hk)
    g = GpuCase(case)
    g.run_steps()
    for kc, vc in oracle_steps(case):
        pass
    ref = oracle_decode(case, kc, vc)
    out = torch.full_like(g.q, float("nan"))
    pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=16)
    st = torch.full_like(g.q, float("nan"))
    pa().decode_static(st, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=16)
    plain = g.decode(out=torch.empty_like(g.q), shared_blocks=True)
    torch.cuda.synchronize()
    assert_close(out, ref, case.dtype, f"{case.name} siblings=16 (split)")
    assert torch.equal(out.view(torch.int16), st.view(torch.int16))
    log(f"{case.name}: max |split siblings - ungrouped| = {(out.float() - plain.float()).abs().max().item():.3e}")


THIN_SHAPES = [
    # dtype, D, B, query heads, K/V heads, prompts, samples, prompt tokens
    ("bf16", 256, 32, 4, 2, 1, 8, 1500),
    ("f16", 64, 8, 16, 4, 2, 8, 1100),
    ("bf16", 128, 16, 16, 2, 1, 4, 2100),  # G = 8: sub-groups of 2
    ("f16", 128, 64, 4, 4, 3, 5, 1300),  # groups cut across prompts
]


@pytest.mark.parametrize("dtype,D,B,H,Hk,prompts,samples,plen", THIN_SHAPES,
                         ids=[f"{t[0]}-D{t[1]}-B{t[2]}-G{t[3] // t[4]}" for t in THIN_SHAPES])
def test_siblings_thin_grid_split_shapes(dtype, D, B, H, Hk, prompts, samples, plen):
    """Split tile lists at other head sizes, block sizes, group sizes and
    dtypes, and with groups that straddle prompts: the oracle's values."""
    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=plen, num_heads=H,
                                head_dim=D, pool_tokens=65536, max_suffix=48, num_kv_heads=Hk, dtype=dtype)
    group = 4 if samples == 5 else samples
    run_case(case, group)


def test_siblings_thin_grid_split_guards():
    """Split tile lists keep the guards: an empty member gives zeros, an
    impossible one NaN, an out-of-pool id in one member's own blocks NaN for
    that member, one in the shared prompt NaN for the whole group; the other
    members match the oracle."""
    case = _thin_case(8)
    g = GpuCase(case)
    g.run_steps()
    for kc, vc in oracle_steps(case):
        pass
    ref = oracle_decode(case, kc, vc)
    ctx = case.context_lens.copy()
    ctx[3] = 0
    ctx[5] = case.max_context_len + 7
    bt = case.block_tables.copy()
    bt[9, (int(ctx[9]) - 1) // case.block_size] = case.num_blocks + 2  # member 9's last (own) block
    out = torch.full_like(g.q, 1.0)
    pa().decode(out, g.q, g.kc, g.vc, torch.from_numpy(bt).cuda(), torch.from_numpy(ctx).cuda(), case.scale,
                case.max_context_len, siblings=16)
    torch.cuda.synchronize()
    assert (out[3].float() == 0).all()
    assert torch.isnan(out[5].float()).all() and torch.isnan(out[9].float()).all()
    keep = [i for i in range(16) if i not in (3, 5, 9)]
    assert_close(out[keep], ref[keep], case.dtype, "split siblings: other members")
    bt = case.block_tables.copy()
    bt[:, 2] = case.num_blocks + 1  # a shared prompt block of the one group
    out = torch.full_like(g.q, 0.0)
    pa().decode(out, g.q, g.kc, g.vc, torch.from_numpy(bt).cuda(), g.ctx, case.scale, case.max_context_len,
                siblings=16)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()


def test_siblings_thin_grid_split_unrelated():
    """A thin split grid whose members share nothing (every token read
    privately), with an empty and a one-token context among them."""
    case = wl.random_case(91, 8, 4, 128, 16, "bf16", ctx=[1500, 1200, 0, 1100, 2000, 1, 1300, 1700], spare_blocks=4)
    g, out, ref = run_case(case, 8, strict=False)
    assert (out[2].float() == 0).all()


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_siblings_scale_zero_and_negative(scale):
    """Scale 0 (every weight equal: the mean of the V rows) and a negative
    scale, through whole sibling tile lists (config 4's shape at 16 prompts)
    and through a split thin grid."""
    for case, group in ((wl.parallel_sampling(block_size=16, num_prompts=16, samples=4, prompt_len=300,
                                              num_heads=8, head_dim=128, pool_tokens=16384, max_suffix=64), 4),
                        (_thin_case(8), 16)):
        case.scale = scale
        g = GpuCase(case)
        g.run_steps()
        for kc, vc in oracle_steps(case):
            pass
        ref = oracle_decode(case, kc, vc)
        out = torch.full_like(g.q, float("nan"))
        pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, scale, case.max_context_len, siblings=group)
        torch.cuda.synchronize()
        assert_close(out, ref, case.dtype, f"{case.name} siblings={group} scale={scale}")


def test_siblings_thin_grid_declined_without_workspace():
    """Where the ungrouped plan needs no workspace (two prompts x 16 samples,
    multi-head: whole contexts) a thin sibling grid has nowhere to put split
    partials: the hint is declined and the call runs the ungrouped plan with
    cached loads, bit for bit."""
    case = _thin_case(32, prompts=2)
    g = GpuCase(case)
    g.run_steps()
    S, H, D = case.q.shape
    assert pa().decode_workspace_size(S, H, D, case.max_context_len) == 0
    for kc, vc in oracle_steps(case):
        pass
    ref = oracle_decode(case, kc, vc)
    out = torch.full_like(g.q, float("nan"))
    pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=16)
    plain = g.decode(out=torch.empty_like(g.q), shared_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    assert_close(out, ref, case.dtype, f"{case.name} siblings=16 (declined)")
