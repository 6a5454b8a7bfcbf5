"""Paged prefill (pa_prefill) on the GPU against the float64 oracle.

Chunked-prefill batches shaped like a LLaMA-7B layer and a LLaMA-3-8B
(grouped-query) layer, a whole-prompt bf16 batch with the chat-like length
mix, a sweep of ragged shapes (chunks of 1 row, chunks crossing 64-row tiles,
whole prompts, block sizes 1..256, groups 1..8), and the invariants:
chunked == whole-prompt rows, single-row chunks == pa_decode, guards.
Every batch is compared with the oracle on every row of every sequence.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import assert_close, log, out_ulp, pa, to_gpu

pytestmark = pytest.mark.gpu


class PrefillRun:
    """A prefill case resident on the GPU, its chunk written by reshape_and_cache."""

    def __init__(self, case: wl.Case):
        self.case = case
        d = case.dtype
        self.q = to_gpu(case.q, d)
        self.kc = to_gpu(case.k_cache, d)
        self.vc = to_gpu(case.v_cache, d)
        self.bt = to_gpu(case.block_tables)
        self.ctx = to_gpu(case.context_lens)
        self.qs = to_gpu(case.query_start)
        st = case.steps[0]
        pa().reshape_and_cache(to_gpu(st.key, d), to_gpu(st.value, d), self.kc, self.vc, to_gpu(st.slot_mapping))
        self.out = torch.full_like(self.q, float("nan"))

    def run(self, max_query_len=None):
        c = self.case
        mq = int(np.diff(c.query_start).max()) if max_query_len is None else max_query_len
        pa().prefill(self.out, self.q, self.kc, self.vc, self.bt, self.ctx, self.qs, c.scale, mq, c.max_context_len)
        torch.cuda.synchronize()
        return self.out


def oracle_pools(case):
    st = case.steps[0]
    return oracle.reshape_and_cache(st.key, st.value, case.k_cache, case.v_cache, st.slot_mapping)


def oracle_rows(case, kc, vc, seqs):
    """Oracle output for the given sequences only, and their packed row indices."""
    seqs = list(seqs)
    qs = case.query_start
    rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
    sub_qs = np.zeros(len(seqs) + 1, dtype=np.int64)
    sub_qs[1:] = np.cumsum([qs[s + 1] - qs[s] for s in seqs])
    ref = oracle.paged_prefill(case.q[rows], kc, vc, case.block_tables[seqs], case.context_lens[seqs], sub_qs,
                               case.scale, case.dtype)
    return ref, rows


def check(case, seqs=None, strict=True, max_query_len=None):
    run = PrefillRun(case)
    log(f"{case.name}: prefill over {case.num_tokens} rows")
    out = run.run(max_query_len)
    kc, vc = oracle_pools(case)
    seqs = range(case.num_seqs) if seqs is None else seqs
    ref, rows = oracle_rows(case, kc, vc, seqs)
    got = out[torch.from_numpy(rows).cuda()]
    assert_close(got, ref, case.dtype, f"{case.name} prefill", strict=strict)
    return run


@pytest.mark.parametrize("which", ["f16-gqa", "bf16"])
def test_prefill_long_cached_prefix(which):
    """Chunks over cached prefixes of 60000 and 65000 tokens (about 1900 and
    2000 key tiles per workgroup, 3763 and 4094 staged block ids against the
    limit of 4096), beside a whole prompt, a 129-row chunk (a 128-row tile
    plus one row) and a 28-row chunk."""
    if which == "f16-gqa":
        case = wl.random_prefill_case(501, [60000, 0, 3000], [200, 300, 129], 4, 128, 16, "f16", num_kv_heads=2)
    else:
        case = wl.random_prefill_case(502, [65000, 100], [500, 28], 2, 64, 16, "bf16")
    check(case, strict=case.dtype == "f16")


def test_prefill_llama7b_chunked():
    check(wl.prefill_config("llama7b"))


def test_prefill_llama3_8b_gqa_chunked():
    check(wl.prefill_config("llama3-8b"))


def test_prefill_whole_prompts_bf16():
    # A whole prompt's first rows attend to a handful of tokens, so |out|
    # reaches ~3 there, where bf16's half-ulp (2^-7 on [2, 4)) exceeds 2e-3:
    # the bound is 2e-3 or one output ulp, as for the short decode contexts.
    check(wl.prefill_config("prompts"), strict=False)


SWEEP = [
    # dtype, H, Hk, D, B, prefix, chunk
    ("f16", 4, 4, 128, 16, [0, 17, 100], [64, 1, 33]),
    ("bf16", 8, 2, 64, 8, [0, 5], [130, 70]),
    ("f16", 4, 1, 64, 1, [3, 0, 40], [1, 200, 9]),
    ("bf16", 2, 2, 128, 32, [31, 32, 33], [1, 32, 65]),
    ("f16", 6, 3, 128, 4, [0], [257]),
    ("bf16", 8, 8, 64, 256, [300, 0], [20, 300]),
    ("f16", 16, 2, 128, 16, [1000, 0, 7], [63, 129, 1]),
    # head_dim 256: 64-row tiles (one 16-row block per wavefront)
    ("f16", 4, 2, 256, 16, [0, 40, 100], [130, 64, 65]),
    ("bf16", 8, 8, 256, 8, [200, 0], [1, 200]),
]


@pytest.mark.parametrize("dtype,H,Hk,D,B,prefix,chunk", SWEEP,
                         ids=[f"{s[0]}-H{s[1]}-Hk{s[2]}-D{s[3]}-B{s[4]}" for s in SWEEP])
def test_prefill_sweep(dtype, H, Hk, D, B, prefix, chunk):
    case = wl.random_prefill_case(len(prefix) * 7 + D + B, prefix, chunk, H, D, B, dtype, num_kv_heads=Hk)
    # Short contexts give |out| near 1-3: 2e-3 or one output ulp, as for decode.
    check(case, strict=False)
    # A generous max_query_len (up to the context bound the ABI allows) only
    # adds workgroups that exit.
    mq = min(int(max(chunk)) + 130, case.max_context_len)
    if mq > max(chunk):
        check(case, strict=False, max_query_len=mq)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, -0.25])
def test_prefill_zero_and_negative_scale(dtype, scale):
    """Scale 0 makes every row the plain mean of the V rows it may see (keys
    past its position must weigh exactly 0, not 0 * inf); a negative scale is
    an ordinary softmax of the negated scores."""
    base = wl.random_prefill_case(91, [0, 37, 5], [40, 70, 1], 4, 128, 16, dtype, num_kv_heads=2)
    check(dataclasses.replace(base, scale=scale), strict=False)


@pytest.mark.parametrize("dtype,H,Hk", [("f16", 8, 8), ("bf16", 16, 4)])
def test_prefill_dispatch_orders_agree_bitwise(dtype, H, Hk):
    """The launch order of the query tiles (unit-major with sequences ranked
    by context length when the chunks fill the launched tiles, the packed
    level order otherwise) changes no row's arithmetic: a generous
    max_query_len, which would launch mostly empty tiles and so flips the
    order, gives identical bits."""
    case = wl.random_prefill_case(1234 + H, [700, 0, 300, 1500, 64], [256, 250, 130, 200, 256], H, 128, 16, dtype,
                                  num_kv_heads=Hk)
    run = PrefillRun(case)
    mq = int(np.diff(case.query_start).max())
    assert 2 * case.num_tokens >= case.num_seqs * ((mq + 127) // 128) * 128  # unit-major
    a = run.run().clone()
    big = 4 * 128 * ((mq + 127) // 128)
    assert big <= case.max_context_len and 2 * case.num_tokens < case.num_seqs * big  # packed
    b = run.run(max_query_len=big).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    kc, vc = oracle_pools(case)
    ref, rows = oracle_rows(case, kc, vc, range(case.num_seqs))
    assert_close(a[torch.from_numpy(rows).cuda()], ref, dtype, f"{case.name} prefill", strict=False)


def test_prefill_chunks_match_whole_prompt():
    """Prefilling a prompt in three chunks gives the rows the whole-prompt
    prefill gives (within one output ulp)."""
    whole = wl.random_prefill_case(41, [0], [300], 8, 128, 16, "f16", num_kv_heads=2)
    run = PrefillRun(whole)
    ref = run.run().clone()
    q = run.q
    for r0, r1 in ((0, 100), (100, 101), (101, 300)):
        ctx = torch.tensor([r1], dtype=torch.int32, device="cuda")
        qs = torch.tensor([0, r1 - r0], dtype=torch.int32, device="cuda")
        out = torch.empty_like(q[r0:r1])
        pa().prefill(out, q[r0:r1].contiguous(), run.kc, run.vc, run.bt, ctx, qs, whole.scale, r1 - r0, 300)
        torch.cuda.synchronize()
        diff = (out.float() - ref[r0:r1].float()).abs().max().item()
        log(f"chunk rows {r0}..{r1 - 1}: max |chunk - whole| = {diff:.3e}")
        assert diff <= 2e-3, diff


def test_prefill_single_rows_match_decode():
    """Chunks of one row are decode queries: pa_prefill and pa_decode agree."""
    case = wl.random_prefill_case(42, [5, 200, 0, 1023], [1, 1, 1, 1], 8, 128, 16, "bf16", num_kv_heads=4)
    run = PrefillRun(case)
    out = run.run()
    dec = torch.empty_like(out)
    pa().decode(dec, run.q, run.kc, run.vc, run.bt, run.ctx, case.scale, case.max_context_len)
    torch.cuda.synchronize()
    diff = (out.float() - dec.float()).abs().max().item()
    log(f"single-row prefill vs decode: max diff {diff:.3e}")
    kc, vc = oracle_pools(case)
    ref, _ = oracle_rows(case, kc, vc, range(case.num_seqs))
    assert_close(out, ref, case.dtype, "single-row prefill", strict=False)
    assert diff <= 2e-3 * 2


def test_prefill_guards():
    """ctx < n gives NaN rows for that sequence only; an out-of-pool block id
    gives NaN for the rows of the tile that needs it; an empty chunk writes
    nothing.  Nothing faults."""
    case = wl.random_prefill_case(43, [10, 0, 4], [5, 70, 3], 4, 64, 8, "f16")
    run = PrefillRun(case)
    kc, vc = oracle_pools(case)
    # Sequence 0: claim ctx 4 < n 5.
    ctx = case.context_lens.copy()
    ctx[0] = 4
    run.ctx = to_gpu(ctx)
    out = run.run()
    qs = case.query_start
    assert torch.isnan(out[qs[0]:qs[1]].float()).all()
    ref, rows = oracle_rows(case, kc, vc, [1, 2])
    assert_close(out[torch.from_numpy(rows).cuda()], ref, case.dtype, "guard: other sequences", strict=False)
    # Sequence 1: an out-of-pool id in its last block.
    run.ctx = to_gpu(case.context_lens)
    bt = case.block_tables.copy()
    nb = -(-int(case.context_lens[1]) // case.block_size)
    bt[1, nb - 1] = case.num_blocks + 5
    run.bt = to_gpu(bt)
    run.out.fill_(0)
    out = run.run()
    rows1 = out[qs[1]:qs[2]].float()
    assert torch.isnan(rows1[-1]).all()  # the last row needs the last block
    ref, rows = oracle_rows(case, kc, vc, [0, 2])
    assert_close(out[torch.from_numpy(rows).cuda()], ref, case.dtype, "guard: bad id elsewhere", strict=False)
    # An empty chunk: sequence 2 with no rows leaves the output untouched.
    qs2 = case.query_start.copy()
    qs2[3] = qs2[2]
    run.bt = to_gpu(case.block_tables)
    run.qs = to_gpu(qs2)
    run.out.fill_(7.0)
    pa().prefill(run.out, run.q, run.kc, run.vc, run.bt, run.ctx, run.qs, case.scale, 70, case.max_context_len)
    torch.cuda.synchronize()
    assert (run.out[qs[2]:qs[3]].float() == 7.0).all()


def test_prefill_tile_major_many_sequences():
    """More than 64 sequences (too many to rank in the kernel) take the
    padded tile-major order; the same chunks prefilled in two calls of at
    most 64 sequences (ranked orders) give identical bits, and every row
    matches the oracle."""
    S = 70
    rng = np.random.default_rng(70)
    prefix = rng.integers(0, 300, S).tolist()
    chunk = rng.integers(1, 200, S).tolist()
    case = wl.random_prefill_case(7070, prefix, chunk, 4, 64, 16, "f16", num_kv_heads=2)
    run = PrefillRun(case)
    whole = run.run().clone()
    kc, vc = oracle_pools(case)
    ref, rows = oracle_rows(case, kc, vc, range(S))
    assert_close(whole[torch.from_numpy(rows).cuda()], ref, "f16", "70-sequence prefill", strict=False)
    qs = case.query_start
    for lo, hi in ((0, 35), (35, 70)):
        r0, r1 = int(qs[lo]), int(qs[hi])
        sub_qs = torch.from_numpy((qs[lo:hi + 1] - r0).astype(np.int32)).cuda()
        out = torch.full_like(run.q[r0:r1], float("nan"))
        pa().prefill(out, run.q[r0:r1].contiguous(), run.kc, run.vc, run.bt[lo:hi].contiguous(),
                     run.ctx[lo:hi].contiguous(), sub_qs, case.scale, int(np.diff(qs).max()), case.max_context_len)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), whole[r0:r1].view(torch.int16)), (lo, hi)


def test_prefill_query_start_guards():
    """Row bounds read from device memory are guarded: a chunk that starts
    below 0 or ends past num_tokens is skipped (its rows keep their old
    contents, nothing faults), and a chunk longer than max_query_len gets
    NaN rows; the other chunks are unaffected."""
    case = wl.random_prefill_case(44, [10, 0, 4, 30], [40, 70, 3, 20], 4, 64, 8, "f16", num_kv_heads=2)
    run = PrefillRun(case)
    kc, vc = oracle_pools(case)
    qs = case.query_start.copy()
    T = case.num_tokens

    def with_qs(new_qs, max_query_len=70):
        run.qs = to_gpu(np.asarray(new_qs, dtype=np.int32))
        run.out.fill_(7.0)
        return run.run(max_query_len=max_query_len)

    def others_match(out, seqs, what):
        ref, rows = oracle_rows(case, kc, vc, seqs)
        assert_close(out[torch.from_numpy(rows).cuda()], ref, case.dtype, what, strict=False)

    # Chunk 0 starts below 0: skipped.
    bad = qs.copy()
    bad[0] = -8
    out = with_qs(bad)
    assert (out[0:qs[1]].float() == 7.0).all()
    others_match(out, [1, 2, 3], "guard: negative start")
    # The last chunk ends past num_tokens: skipped.
    bad = qs.copy()
    bad[-1] = T + 9
    out = with_qs(bad)
    assert (out[qs[3]:T].float() == 7.0).all()
    others_match(out, [0, 1, 2], "guard: end past num_tokens")
    # Chunk 1 (70 rows) is longer than max_query_len = 50: NaN rows.
    out = with_qs(qs, max_query_len=50)
    assert torch.isnan(out[qs[1]:qs[2]].float()).all()
    others_match(out, [0, 2, 3], "guard: chunk longer than max_query_len")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_large_v_rows(dtype):
    """Large V rows.  (a) A common offset of 300 plus small noise under a
    peaked softmax: the offset cancels exactly against the row sum, so every
    element is within 2e-3 or one output ulp.  (b) Rows of +-64 that cancel:
    fp16 probabilities are rounded once to fp16 (relative error <= 2^-11
    each, the row sum taken over the same rounded values), which bounds the
    error by 2^-11 * sum_t w_t |V_t - out| (w the softmax weights); bf16
    probabilities keep a hi/lo split, within 2e-3 or one ulp."""
    base = wl.random_prefill_case(45, [0, 100, 700], [160, 130, 200], 4, 128, 16, dtype, num_kv_heads=2)
    rng = np.random.default_rng(46)
    nb, Hk, B, D = base.v_cache.shape

    def store(x):
        return wl.to_storage(x.astype(np.float32), dtype)

    def prefill_with_v(v_fn, q_gain, strict_ok):
        v = v_fn((nb, Hk, B, D))
        c = dataclasses.replace(base, v_cache=store(v), q=store(oracle.widen(base.q, dtype) * q_gain))
        c.steps = list(c.steps)
        st = c.steps[0]
        st_v = store(v_fn(st.value.shape))
        c.steps[0] = dataclasses.replace(st, value=st_v)
        run = PrefillRun(c)
        out = run.run()
        kc2, vc2 = oracle_pools(c)
        ref, rows = oracle_rows(c, kc2, vc2, range(c.num_seqs))
        got = out[torch.from_numpy(rows).cuda()]
        if strict_ok:
            assert_close(got, ref, dtype, f"{dtype} large V", strict=False)
            return
        # Proven bound for one rounded fp16 probability operand: each
        # probability p (<= 2^8, relative to a reference that makes the row's
        # sum >= 1) is off by at most 2^-11 p, or 2^-25 where fp16 is
        # subnormal; the output moves by sum_t (p~_t - p_t)(V_t - out) / sum_t p_t.
        wdev, adev = oracle_v_spread(c, kc2, vc2)
        bound = wdev * 2.0 ** -11 + adev * 2.0 ** -25
        err = np.abs(got.double().cpu().numpy() - ref)
        ulp = out_ulp(ref, dtype)
        log(f"{dtype} cancelling V: max err {err.max():.3e}, max err / bound {(err / (bound + ulp)).max():.3f}")
        assert (err <= bound + ulp).all()

    # (a) offset 300 + N(0, 0.25) noise, peaked softmax (queries x 4).
    prefill_with_v(lambda shp: 300.0 + 0.5 * rng.standard_normal(shp), 4.0, True)
    # (b) +-64 rows that cancel, moderately peaked softmax.
    signs = lambda shp: 64.0 * np.where(rng.random(shp) < 0.5, -1.0, 1.0) + rng.standard_normal(shp)
    prefill_with_v(signs, 2.0, dtype == "bf16")


def oracle_v_spread(case, kc, vc):
    """Per (row, head, channel): sum_t w_t |V_t - out| (the weighted mean
    deviation of the attended V rows from the output, w the softmax
    weights) and sum_t |V_t - out|, in float64."""
    qs = case.query_start
    T, H, D = case.q.shape
    Hk = case.k_cache.shape[1]
    G = H // Hk
    spread = np.zeros((T, H, D))
    total = np.zeros((T, H, D))
    for s in range(case.num_seqs):
        r0, r1 = int(qs[s]), int(qs[s + 1])
        n, ctx = r1 - r0, int(case.context_lens[s])
        K = oracle.widen(oracle.logical_kv(kc, case.block_tables[s], ctx), case.dtype)
        V = oracle.widen(oracle.logical_kv(vc, case.block_tables[s], ctx), case.dtype)
        Q = oracle.widen(case.q[r0:r1], case.dtype)
        for h in range(H):
            for i in range(n):
                p = ctx - n + i
                sc = case.scale * (K[h // G, : p + 1] @ Q[i, h])
                w = np.exp(sc - sc.max())
                w /= w.sum()
                o = w @ V[h // G, : p + 1]
                dev = np.abs(V[h // G, : p + 1] - o)
                spread[r0 + i, h] = w @ dev
                total[r0 + i, h] = dev.sum(axis=0)
    return spread, total

