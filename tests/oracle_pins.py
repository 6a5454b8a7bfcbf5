"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes the oracle module and raises AssertionError if
the oracle disagrees with an independent fact: brute force over the
per-token definition, a library attention routine, closed forms, invariants,
the block-table layouts the pages draw, and round trips.  They are shared by
``test_oracle_pins.py`` (the real oracle must pass all of them) and
``test_oracle_mutations.py`` (an oracle with a planted mistake must fail at
least one of them).
"""
from __future__ import annotations

import functools
import json
import math
import os

import numpy as np
import torch

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@functools.lru_cache(None)
def _opt13b():
    return wl.opt13b_decode()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Independent helpers (never call the oracle)
# ---------------------------------------------------------------------------


def torch_widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Float64 value of stored elements, decoded by torch's own casts."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.double().numpy()


def brute_decode(q, kc, vc, bt, ctx, scale, dtype) -> np.ndarray:
    """Per-token loops over the definition: for each query, each context
    token t is found at physical block bt[s][t // B], offset t % B; score =
    scale * sum_d q_d k_d (math.fsum); softmax with math.exp; weighted V sum
    with math.fsum.  Slow, tiny inputs only."""
    qw, kw, vw = torch_widen(q, dtype), torch_widen(kc, dtype), torch_widen(vc, dtype)
    S, H, D = q.shape
    B = kc.shape[2]
    G = H // kc.shape[1]  # query heads per K/V head
    out = np.zeros((S, H, D))
    for s in range(S):
        n = int(ctx[s])
        if n <= 0:
            continue
        loc = [(int(bt[s][t // B]), t % B) for t in range(n)]
        for h in range(H):
            hk = h // G
            sc = [scale * math.fsum(float(qw[s, h, d]) * float(kw[b, hk, o, d]) for d in range(D)) for b, o in loc]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            z = math.fsum(e)
            for d in range(D):
                out[s, h, d] = math.fsum(e[t] * float(vw[b, hk, o, d]) for t, (b, o) in enumerate(loc)) / z
    return out


def scatter_contiguous(K: np.ndarray, table, B: int, N: int, dtype: str):
    """Build an [N, H, B, D] pool holding contiguous K [H, n, D] at the blocks
    named by ``table`` (token t -> block table[t // B], slot t % B), by loops.
    Unused slots hold canaries."""
    H, n, D = K.shape
    pool = wl.canary_fill((N, H, B, D), dtype)
    for t in range(n):
        b, o = table[t // B], t % B
        for h in range(H):
            pool[b, h, o, :] = K[h, t, :]
    return pool


def _decode(orc, case: wl.Case, q=None, kc=None, vc=None, bt=None, ctx=None, scale=None):
    return orc.paged_decode(
        case.q if q is None else q,
        case.k_cache if kc is None else kc,
        case.v_cache if vc is None else vc,
        case.block_tables if bt is None else bt,
        case.context_lens if ctx is None else ctx,
        case.scale if scale is None else scale,
        case.dtype,
    )


def _small_cases():
    yield wl.tiny_f32()
    yield wl.random_case(1, 4, 2, 8, 4, "f32", ctx_range=(1, 21))
    yield wl.random_case(2, 3, 2, 4, 2, "f16", ctx_range=(1, 13))
    yield wl.random_case(3, 3, 1, 8, 3, "bf16", ctx_range=(1, 17))
    yield wl.random_case(4, 2, 2, 8, 1, "f32", ctx=[1, 9])
    yield wl.random_case(5, 3, 2, 8, 4, "bf16", ctx=[0, 4, 11])
    yield wl.random_case(18, 3, 4, 8, 4, "f16", ctx=[3, 9, 14], num_kv_heads=2)
    yield wl.random_case(19, 2, 4, 4, 2, "f32", ctx=[5, 1], num_kv_heads=1)


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------


def pin_widen(orc):
    """Stored f16/bf16/f32 values widen exactly as torch decodes them."""
    rng = np.random.default_rng(11)
    for dtype in wl.DTYPES:
        bits = rng.integers(0, 2 ** (8 * wl.ELEM_BYTES[dtype]), 4096, dtype=np.uint64)
        a = bits.astype(wl.NP_BITS[dtype]).view(wl.NP_STORAGE[dtype])
        ref = torch_widen(a, dtype)
        got = orc.widen(a, dtype)
        fin = np.isfinite(ref)
        assert np.array_equal(got[fin], ref[fin]), dtype
        assert np.array_equal(np.isnan(got), np.isnan(ref)), dtype


def pin_bruteforce(orc):
    """Vectorised oracle == per-token brute force on tiny cases (<= 1e-12)."""
    for case in _small_cases():
        got = _decode(orc, case)
        ref = brute_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale, case.dtype)
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (case.name, err)


def pin_library_attention(orc):
    """With K/V scattered into a pool by explicit loops, the paged result
    equals torch's scaled_dot_product_attention on the contiguous tensors."""
    rng = np.random.default_rng(12)
    for dtype, H, D, B, n in (("f32", 3, 16, 8, 37), ("f16", 2, 32, 4, 29), ("bf16", 4, 8, 16, 16), ("f32", 2, 8, 2, 1)):
        nb = -(-n // B)
        N = nb + 4
        table = rng.permutation(N)[:nb]
        K = wl.to_storage(rng.standard_normal((H, n, D), dtype=np.float32), dtype)
        V = wl.to_storage(rng.standard_normal((H, n, D), dtype=np.float32), dtype)
        q = wl.to_storage(rng.standard_normal((1, H, D), dtype=np.float32), dtype)
        kc = scatter_contiguous(K, table, B, N, dtype)
        vc = scatter_contiguous(V, table, B, N, dtype)
        bt = np.full((1, nb + 2), -1, dtype=np.int32)
        bt[0, :nb] = table
        scale = 1.0 / math.sqrt(D)
        got = orc.paged_decode(q, kc, vc, bt, np.array([n], np.int32), scale, dtype)
        tq = torch.from_numpy(torch_widen(q, dtype)).reshape(1, H, 1, D)
        tk = torch.from_numpy(torch_widen(K, dtype)).unsqueeze(0)
        tv = torch.from_numpy(torch_widen(V, dtype)).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).reshape(1, H, D).numpy()
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (dtype, err)
        # Plain softmax attention written with torch ops, too.
        w = torch.softmax(scale * (tk[0] @ tq[0].transpose(1, 2)).squeeze(-1), dim=-1)
        ref2 = (w.unsqueeze(1) @ tv[0]).squeeze(1).numpy()
        assert np.abs(got[0] - ref2).max() <= 1e-12


def pin_permutation(orc):
    """Relabelling physical blocks (moving them and rewriting the tables)
    leaves the result bit-for-bit unchanged."""
    rng = np.random.default_rng(13)
    for case in (wl.tiny_f32(), wl.random_case(6, 4, 2, 8, 4, "f16", ctx_range=(1, 30)), wl.random_case(7, 3, 2, 8, 2, "bf16")):
        base = _decode(orc, case)
        pi = rng.permutation(case.num_blocks)
        kc = np.empty_like(case.k_cache)
        vc = np.empty_like(case.v_cache)
        kc[pi] = case.k_cache
        vc[pi] = case.v_cache
        bt = np.where(case.block_tables >= 0, pi[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
        got = _decode(orc, case, kc=kc, vc=vc, bt=bt)
        assert np.array_equal(got, base), case.name


def pin_single_token(orc):
    """A context of one token returns that token's V row exactly."""
    for dtype in wl.DTYPES:
        case = wl.random_case(8, 3, 2, 8, 4, dtype, ctx=[1, 1, 1])
        got = _decode(orc, case)
        for s in range(3):
            b = case.block_tables[s, 0]
            assert np.array_equal(got[s], torch_widen(case.v_cache[b, :, 0, :], dtype)), dtype


def pin_closed_forms(orc):
    """scale 0 or K = 0 -> mean of V rows; equal V rows -> that row;
    two tokens -> logistic weights; empty context -> zeros."""
    case = wl.random_case(9, 2, 2, 8, 4, "f32", ctx=[7, 13])
    vmean = []
    for s in range(2):
        n = int(case.context_lens[s])
        rows = [case.v_cache[case.block_tables[s][t // 4], :, t % 4, :].astype(np.float64) for t in range(n)]
        vmean.append(np.array([[math.fsum(r[h, d] for r in rows) / n for d in range(8)] for h in range(2)]))
    vmean = np.stack(vmean)
    assert np.abs(_decode(orc, case, scale=0.0) - vmean).max() <= 1e-14
    kz = np.where(np.isnan(case.k_cache), case.k_cache, np.float32(0))
    assert np.abs(_decode(orc, case, kc=kz) - vmean).max() <= 1e-14
    # Every token of a (sequence, head) has the same V row c -> output c.
    vconst = case.v_cache.copy()
    c = np.arange(1, 9, dtype=np.float32) / 8
    for s in range(2):
        for t in range(int(case.context_lens[s])):
            vconst[case.block_tables[s][t // 4], :, t % 4, :] = c * (1 + s)
    got = _decode(orc, case, vc=vconst)
    for s in range(2):
        assert np.abs(got[s] - (c * (1 + s)).astype(np.float64)).max() <= 1e-14
    # Two tokens: weight of token 0 is the logistic function of the score gap.
    two = wl.random_case(10, 1, 3, 8, 4, "f32", ctx=[2], scale=0.7)
    qv = two.q[0].astype(np.float64)
    b = two.block_tables[0, 0]
    k0, k1 = two.k_cache[b, :, 0, :].astype(np.float64), two.k_cache[b, :, 1, :].astype(np.float64)
    v0, v1 = two.v_cache[b, :, 0, :].astype(np.float64), two.v_cache[b, :, 1, :].astype(np.float64)
    gap = 0.7 * (np.sum(qv * k0, axis=1) - np.sum(qv * k1, axis=1))
    w0 = 1.0 / (1.0 + np.exp(-gap))
    ref = w0[:, None] * v0 + (1.0 - w0)[:, None] * v1
    assert np.abs(_decode(orc, two)[0] - ref).max() <= 1e-13
    # Empty context (reading: zero output).
    empty = wl.random_case(11, 2, 1, 8, 4, "f16", ctx=[0, 3])
    assert np.array_equal(_decode(orc, empty)[0], np.zeros((1, 8)))


def _marker_pool(N, B):
    """Pool whose slot (block b, offset o) holds the vector [b, o, 0, 0]."""
    kc = np.zeros((N, 1, B, 4), dtype=np.float32)
    for b in range(N):
        for o in range(B):
            kc[b, 0, o, 0] = b
            kc[b, 0, o, 1] = o
    return kc


def pin_page_layouts(orc):
    """The block tables drawn on the pages resolve tokens to the drawn blocks."""
    g = _golden("digest_flowchart_layout.json")
    B, N = g["block_size"], g["pool_blocks"]
    pool = _marker_pool(N, B)
    for seq, n_list in g["lengths"].items():
        table = np.array(g["tables"][seq], dtype=np.int32)
        for n in n_list:
            assert orc.blocks_held(n, B) == g["blocks_held"][seq]
            kv = orc.logical_kv(pool, table, n)
            for j, (lo, hi) in enumerate(g["logical_block_token_ranges"][seq]):
                hi = n - 1 if hi is None else hi
                for t in range(lo, hi + 1):
                    assert kv[0, t, 0] == table[j] and kv[0, t, 1] == t - lo
    for loc in g["token_locations"]:
        table = np.array(g["tables"][loc["seq"]], dtype=np.int32)
        assert orc.token_location(table, loc["token"], B) == (loc["block"], loc["offset"])
        kv = orc.logical_kv(pool, table, loc["token"] + 1)
        assert (kv[0, loc["token"], 0], kv[0, loc["token"], 1]) == (loc["block"], loc["offset"])

    # Copy-on-write of the shared block P3 into the free P9.
    rng = np.random.default_rng(14)
    H, D = 2, 8
    kc = wl.canary_fill((N, H, B, D), "f32")
    vc = wl.canary_fill((N, H, B, D), "f32")
    lens = {"seq1": 33, "seq2": 17}
    for seq, n in lens.items():
        for t in range(n):
            b = g["tables"][seq][t // B]
            kc[b, :, t % B, :] = rng.standard_normal((H, D))
            vc[b, :, t % B, :] = rng.standard_normal((H, D))
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    bt = np.full((2, 3), -1, dtype=np.int32)
    bt[0, :3] = g["tables"]["seq1"]
    bt[1, :2] = g["tables"]["seq2"]
    ctx = np.array([lens["seq1"], lens["seq2"]], dtype=np.int32)
    before = orc.paged_decode(q, kc, vc, bt, ctx, 0.5, "f32")
    src, dst = g["cow"]["src"], g["cow"]["dst"]
    kc2, vc2 = orc.copy_blocks(kc, vc, [(src, dst)])
    assert np.array_equal(kc2[dst].view(np.uint32), kc[src].view(np.uint32))
    assert np.array_equal(vc2[dst].view(np.uint32), vc[src].view(np.uint32))
    bt2 = bt.copy()
    bt2[1, 0] = dst
    after = orc.paged_decode(q, kc2, vc2, bt2, ctx, 0.5, "f32")
    assert np.array_equal(before, after)
    # A divergent write into sequence 2's private copy leaves sequence 1 alone.
    kn = rng.standard_normal((1, H, D)).astype(np.float32)
    vn = rng.standard_normal((1, H, D)).astype(np.float32)
    kc3, vc3 = orc.reshape_and_cache(kn, vn, kc2, vc2, np.array([dst * B + 5], dtype=np.int64))
    div = orc.paged_decode(q, kc3, vc3, bt2, ctx, 0.5, "f32")
    assert np.array_equal(div[0], before[0])
    assert not np.array_equal(div[1], before[1])

    v = _golden("velog_block_table.json")
    pool = _marker_pool(v["pool_blocks"], v["block_size"])
    kv = orc.logical_kv(pool, np.array(v["table"], dtype=np.int32), len(v["table"]) * v["block_size"])
    for t in range(kv.shape[1]):
        assert kv[0, t, 0] == v["table"][t // v["block_size"]] and kv[0, t, 1] == t % v["block_size"]

    for c in _golden("blocks_needed.json")["cases"]:
        nb = orc.blocks_held(c["tokens"], c["block_size"])
        assert nb == c["blocks"]
        assert nb * c["block_size"] - c["tokens"] == c["last_block_free_slots"]


def pin_append(orc):
    """Appending writes each token's rows exactly where the block table says,
    reading the sequence back returns them bit-exactly, and nothing else in
    the pool changes; negative slots are skipped."""
    for dtype in wl.DTYPES:
        case = wl.random_case(15, 4, 3, 8, 4, dtype, ctx_range=(3, 23), n_append=3, spare_blocks=5)
        st = case.steps[0]
        slots = st.slot_mapping.copy()
        slots[1] = -1  # padding token
        kc, vc = orc.reshape_and_cache(st.key, st.value, case.k_cache, case.v_cache, slots)
        B = case.block_size
        written = np.zeros(case.k_cache.shape[:1] + case.k_cache.shape[2:3], dtype=bool)
        for i, sl in enumerate(slots):
            if sl < 0:
                continue
            b, o = int(sl) // B, int(sl) % B
            written[b, o] = True
            assert np.array_equal(wl.bits_view(kc[b, :, o, :]), wl.bits_view(st.key[i]))
            assert np.array_equal(wl.bits_view(vc[b, :, o, :]), wl.bits_view(st.value[i]))
        keep = ~written
        assert np.array_equal(wl.bits_view(kc).transpose(0, 2, 1, 3)[keep], wl.bits_view(case.k_cache).transpose(0, 2, 1, 3)[keep])
        assert np.array_equal(wl.bits_view(vc).transpose(0, 2, 1, 3)[keep], wl.bits_view(case.v_cache).transpose(0, 2, 1, 3)[keep])
        # Read back through the block table: the new tokens are the last ones.
        n_new = 3
        for s in range(case.num_seqs):
            n = int(case.context_lens[s])
            kv = orc.logical_kv(kc, case.block_tables[s], n)
            for r in range(n_new):
                i = s * n_new + r
                if slots[i] < 0:
                    continue
                assert np.array_equal(wl.bits_view(kv[:, n - n_new + r, :]), wl.bits_view(st.key[i]))


def pin_cow(orc):
    """Block copies: destination equals source bit-for-bit, other blocks are
    untouched, reading through a copy gives the same attention as through the
    original, and a write into one sample's block does not reach the others."""
    case = wl.parallel_sampling(block_size=4, num_prompts=3, samples=4, prompt_len=10, num_heads=2, head_dim=8, pool_tokens=4096)
    ap0, cp, ap1 = case.steps
    kc, vc = orc.reshape_and_cache(ap0.key, ap0.value, case.k_cache, case.v_cache, ap0.slot_mapping)
    kc2, vc2 = orc.copy_blocks(kc, vc, cp.pairs)
    assert cp.pairs.shape == (9, 2)
    moved = np.zeros(case.num_blocks, dtype=bool)
    for src, dst in cp.pairs:
        moved[dst] = True
        assert np.array_equal(wl.bits_view(kc2[dst]), wl.bits_view(kc[src]))
        assert np.array_equal(wl.bits_view(vc2[dst]), wl.bits_view(vc[src]))
    assert np.array_equal(wl.bits_view(kc2[~moved]), wl.bits_view(kc[~moved]))
    assert np.array_equal(wl.bits_view(vc2[~moved]), wl.bits_view(vc[~moved]))
    # Before any suffix write, every sample (copy or original) sees the prompt.
    pre_ctx = np.full(case.num_seqs, 10, dtype=np.int32)
    fork_out = orc.paged_decode(case.q, kc2, vc2, case.block_tables, pre_ctx, case.scale, case.dtype)
    orig_bt = case.block_tables.copy()
    for g in range(3):
        orig_bt[4 * g : 4 * g + 4] = case.block_tables[4 * g + 3]
    base_out = orc.paged_decode(case.q, kc2, vc2, orig_bt, pre_ctx, case.scale, case.dtype)
    assert np.array_equal(fork_out, base_out)
    # After the suffix writes, samples 0..2 still read the unchanged prompt
    # tokens; sample 3 wrote into the original last block in place.
    kc3, vc3 = orc.reshape_and_cache(ap1.key, ap1.value, kc2, vc2, ap1.slot_mapping)
    for g in range(3):
        last = 10 // 4
        orig = case.block_tables[4 * g + 3, last]
        for i in range(3):
            mine = case.block_tables[4 * g + i, last]
            assert mine != orig
            for o in range(10 % 4):
                assert np.array_equal(wl.bits_view(kc3[mine, :, o]), wl.bits_view(kc[orig, :, o]))
    out = orc.paged_decode(case.q, kc3, vc3, case.block_tables, case.context_lens, case.scale, case.dtype)
    ref = brute_decode(case.q, kc3, vc3, case.block_tables, case.context_lens, case.scale, case.dtype)
    assert np.abs(out - ref).max() <= 1e-12


def pin_split_merge(orc):
    """Merging the partials of any split of the context reproduces the
    unsplit attention, and one slice's o / l is its own attention."""
    rng = np.random.default_rng(16)
    for n in (1, 5, 64, 333):
        q = rng.standard_normal(16)
        K = rng.standard_normal((n, 16)) * 2
        V = rng.standard_normal((n, 16))
        full = orc.attention(q, K, V, 0.3)
        # Independent reference: softmax with math.fsum.
        sc = [0.3 * math.fsum(q * K[t]) for t in range(n)]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        ref = np.array([math.fsum(e[t] * V[t, d] for t in range(n)) for d in range(16)]) / math.fsum(e)
        assert np.abs(full - ref).max() <= 1e-13
        for _ in range(3):
            cuts = sorted(set(rng.integers(1, n, size=min(4, max(0, n - 1))).tolist())) if n > 1 else []
            bounds = [0] + cuts + [n]
            parts = [orc.partial_attention(q, K[a:b], V[a:b], 0.3) for a, b in zip(bounds[:-1], bounds[1:])]
            assert np.abs(orc.merge_partials(parts) - ref).max() <= 1e-13
            m, l, o = parts[0]
            a, b = bounds[0], bounds[1]
            assert np.abs(o / l - orc.attention(q, K[a:b], V[a:b], 0.3)).max() <= 1e-13
        # A slice whose scores are far below the others contributes ~nothing.
        parts = [orc.partial_attention(q, K, V, 0.3), (-1e4, 1.0, np.full(16, 7.0))]
        assert np.abs(orc.merge_partials(parts) - ref).max() <= 1e-13


def pin_newest_token_slots(orc):
    """The newest token's slot agrees with the slots the host block pool
    handed out when that token was appended (workloads built independently of
    the oracle), with the Digest flowchart's tables, and with ctx <= 0 -> -1;
    append_decode equals append followed by decode."""
    case = _opt13b()
    st = case.steps[0]
    assert np.array_equal(orc.newest_token_slots(case.block_tables, case.context_lens, 16), st.slot_mapping)
    g = _golden("digest_flowchart_layout.json")
    bt = np.full((2, 3), -1, dtype=np.int32)
    bt[0, :3] = g["tables"]["seq1"]
    bt[1, :2] = g["tables"]["seq2"]
    # Seq1 with 33 tokens: token 32 is the first of block 2 (P1); Seq2 with 17: token 16 opens block 1 (P5).
    assert orc.newest_token_slots(bt, np.array([33, 17]), 16).tolist() == [1 * 16 + 0, 5 * 16 + 0]
    assert orc.newest_token_slots(bt, np.array([48, 0]), 16).tolist() == [1 * 16 + 15, -1]
    small = wl.random_case(17, 4, 2, 8, 4, "bf16", ctx_range=(1, 30), n_append=1)
    sa = small.steps[0]
    out, kc, vc = orc.append_decode(small.q, sa.key, sa.value, small.k_cache, small.v_cache, small.block_tables,
                                    small.context_lens, small.scale, small.dtype)
    ref = brute_decode(small.q, *orc.reshape_and_cache(sa.key, sa.value, small.k_cache, small.v_cache,
                                                       sa.slot_mapping), small.block_tables, small.context_lens,
                       small.scale, small.dtype)
    assert np.abs(out - ref).max() <= 1e-12
    assert np.array_equal(wl.bits_view(kc), wl.bits_view(orc.reshape_and_cache(
        sa.key, sa.value, small.k_cache, small.v_cache, sa.slot_mapping)[0]))


def pin_grouped_query(orc):
    """Grouped-query attention: the same as multi-head attention over a cache
    whose K/V heads are each repeated G times, and the same as torch's
    scaled_dot_product_attention with enable_gqa on the contiguous tensors."""
    for dtype, H, Hk in (("f32", 8, 2), ("bf16", 6, 3), ("f16", 4, 1), ("f32", 4, 4)):
        case = wl.random_case(20 + H + Hk, 3, H, 16, 4, dtype, ctx_range=(1, 30), num_kv_heads=Hk)
        G = H // Hk
        got = _decode(orc, case)
        kc = np.repeat(case.k_cache, G, axis=1)  # head h of the copy = K/V head h // G
        vc = np.repeat(case.v_cache, G, axis=1)
        assert np.array_equal(got, _decode(orc, case, kc=kc, vc=vc)), (dtype, H, Hk)
        for s in range(case.num_seqs):
            n = int(case.context_lens[s])
            rows_k = np.stack([case.k_cache[case.block_tables[s][t // 4], :, t % 4, :] for t in range(n)], axis=1)
            rows_v = np.stack([case.v_cache[case.block_tables[s][t // 4], :, t % 4, :] for t in range(n)], axis=1)
            tq = torch.from_numpy(torch_widen(case.q[s], dtype)).reshape(1, H, 1, 16)
            tk = torch.from_numpy(torch_widen(rows_k, dtype)).unsqueeze(0)
            tv = torch.from_numpy(torch_widen(rows_v, dtype)).unsqueeze(0)
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=case.scale, enable_gqa=True)
            assert np.abs(got[s] - ref.reshape(H, 16).numpy()).max() <= 1e-12


ALL_PINS = [
    pin_widen,
    pin_bruteforce,
    pin_library_attention,
    pin_permutation,
    pin_single_token,
    pin_closed_forms,
    pin_page_layouts,
    pin_append,
    pin_cow,
    pin_split_merge,
    pin_newest_token_slots,
    pin_grouped_query,
]


# ---------------------------------------------------------------------------
# Prefill pins (take the oracle.prefill module)
# ---------------------------------------------------------------------------


def brute_prefill(q, kc, vc, bt, ctx, query_start, scale, dtype) -> np.ndarray:
    """Per-token loops over the prefill definition: row i of sequence s sits
    at position ctx_s - n_s + i and attends to positions 0 .. that position;
    token t is found at block bt[s][t // B], slot t % B.  math.fsum sums,
    math.exp weights.  Tiny inputs only."""
    qw, kw, vw = torch_widen(q, dtype), torch_widen(kc, dtype), torch_widen(vc, dtype)
    T, H, D = q.shape
    B = kc.shape[2]
    G = H // kc.shape[1]
    out = np.zeros((T, H, D))
    for s in range(len(ctx)):
        r0, r1 = int(query_start[s]), int(query_start[s + 1])
        n, c = r1 - r0, int(ctx[s])
        for i in range(n):
            pos = c - n + i
            loc = [(int(bt[s][t // B]), t % B) for t in range(pos + 1)]
            for h in range(H):
                hk = h // G
                sc = [scale * math.fsum(float(qw[r0 + i, h, d]) * float(kw[b, hk, o, d]) for d in range(D))
                      for b, o in loc]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                z = math.fsum(e)
                for d in range(D):
                    out[r0 + i, h, d] = math.fsum(e[t] * float(vw[b, hk, o, d]) for t, (b, o) in enumerate(loc)) / z
    return out


def _prefill_small_cases():
    yield wl.random_prefill_case(1, [0, 5, 17], [3, 1, 20], 2, 8, 4, "f32")
    yield wl.random_prefill_case(2, [0, 0], [7, 1], 2, 4, 2, "f16")
    yield wl.random_prefill_case(3, [9, 2, 0, 4], [2, 6, 5, 1], 4, 8, 3, "bf16", num_kv_heads=2)
    yield wl.random_prefill_case(4, [1], [12], 4, 4, 1, "f32", num_kv_heads=1)


def _prefill_pools(case):
    """Pools after the case's chunk is written, by explicit loops (no oracle)."""
    kc, vc = case.k_cache.copy(), case.v_cache.copy()
    B = kc.shape[2]
    for st in case.steps:
        for i, slot in enumerate(st.slot_mapping):
            b, o = int(slot) // B, int(slot) % B
            kc[b, :, o, :] = st.key[i]
            vc[b, :, o, :] = st.value[i]
    return kc, vc


def _prefill(orc, case, kc, vc, q=None, ctx=None, qs=None, scale=None):
    return orc.paged_prefill(case.q if q is None else q, kc, vc, case.block_tables,
                             case.context_lens if ctx is None else ctx,
                             case.query_start if qs is None else qs,
                             case.scale if scale is None else scale, case.dtype)


def pin_prefill_bruteforce(orp):
    """Prefill oracle == per-token brute force on tiny ragged paged cases,
    incl. whole prompts (no prefix), single-row chunks, B = 1 and groups."""
    for case in _prefill_small_cases():
        kc, vc = _prefill_pools(case)
        got = _prefill(orp, case, kc, vc)
        ref = brute_prefill(case.q, kc, vc, case.block_tables, case.context_lens, case.query_start, case.scale,
                            case.dtype)
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (case.name, err)


def pin_prefill_library(orp):
    """Contiguous K/V scattered into a pool by loops: a whole-prompt prefill
    equals torch's causal scaled_dot_product_attention, and a chunk after a
    prefix equals the last rows of that causal attention over the whole
    sequence (torch aligns its causal mask to the first query, so the chunk's
    offset is checked against an independent placement)."""
    rng = np.random.default_rng(21)
    for dtype, H, Hk, D, B, ctx, n in (("f32", 2, 2, 16, 4, 23, 23), ("f16", 4, 2, 32, 8, 40, 13),
                                       ("bf16", 2, 1, 8, 16, 17, 1), ("f32", 3, 3, 8, 2, 9, 5)):
        nb = -(-ctx // B)
        N = nb + 3
        table = rng.permutation(N)[:nb]
        K = wl.to_storage(rng.standard_normal((Hk, ctx, D), dtype=np.float32), dtype)
        V = wl.to_storage(rng.standard_normal((Hk, ctx, D), dtype=np.float32), dtype)
        Qall = wl.to_storage(rng.standard_normal((ctx, H, D), dtype=np.float32), dtype)
        kc = scatter_contiguous(K, table, B, N, dtype)
        vc = scatter_contiguous(V, table, B, N, dtype)
        bt = np.full((1, nb + 1), -1, dtype=np.int32)
        bt[0, :nb] = table
        scale = 1.0 / math.sqrt(D)
        q = np.ascontiguousarray(Qall[ctx - n:])
        got = orp.paged_prefill(q, kc, vc, bt, np.array([ctx], np.int32), np.array([0, n], np.int32), scale, dtype)
        G = H // Hk
        tq = torch.from_numpy(torch_widen(Qall, dtype)).permute(1, 0, 2).unsqueeze(0)  # [1, H, ctx, D]
        tk = torch.from_numpy(torch_widen(K, dtype)).repeat_interleave(G, dim=0).unsqueeze(0)
        tv = torch.from_numpy(torch_widen(V, dtype)).repeat_interleave(G, dim=0).unsqueeze(0)
        full = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
        ref = full[0].permute(1, 0, 2).numpy()[ctx - n:]
        err = np.abs(got - ref).max()
        assert err <= 1e-12, (dtype, H, Hk, ctx, n, err)


def pin_prefill_single_query(orp):
    """Chunks of one row are decode queries: the result equals the
    brute-force decode of the same queries over the same contexts."""
    case = wl.random_prefill_case(5, [4, 0, 11], [1, 1, 1], 4, 8, 4, "f16", num_kv_heads=2)
    kc, vc = _prefill_pools(case)
    got = _prefill(orp, case, kc, vc)
    ref = brute_decode(case.q, kc, vc, case.block_tables, case.context_lens, case.scale, case.dtype)
    assert np.abs(got - ref).max() <= 1e-12


def pin_prefill_chunking(orp):
    """Prefilling a prompt in chunks gives each row exactly the value the
    whole-prompt prefill gives it (a row depends only on its position)."""
    case = wl.random_prefill_case(6, [0], [21], 2, 8, 4, "bf16")
    kc, vc = _prefill_pools(case)
    whole = _prefill(orp, case, kc, vc)
    for cuts in ((5, 21), (1, 2, 21), (20, 21)):
        r0 = 0
        for r1 in cuts:
            part = orp.paged_prefill(case.q[r0:r1], kc, vc, case.block_tables, np.array([r1], np.int32),
                                     np.array([0, r1 - r0], np.int32), case.scale, case.dtype)
            assert np.array_equal(part, whole[r0:r1]), cuts
            r0 = r1


def pin_prefill_closed_forms(orp):
    """scale = 0: the row at position p is the mean of V rows 0 .. p (a
    running mean); the first row of a whole prompt is V row 0 exactly."""
    case = wl.random_prefill_case(7, [3, 0], [6, 5], 2, 8, 4, "f32")
    kc, vc = _prefill_pools(case)
    got = _prefill(orp, case, kc, vc, scale=0.0)
    B = kc.shape[2]
    vw = torch_widen(vc, "f32")
    for s in range(case.num_seqs):
        r0, r1 = int(case.query_start[s]), int(case.query_start[s + 1])
        n, c = r1 - r0, int(case.context_lens[s])
        rows = np.stack([vw[int(case.block_tables[s][t // B]), :, t % B, :] for t in range(c)])  # [c, H, D]
        run_mean = np.cumsum(rows, axis=0) / np.arange(1, c + 1)[:, None, None]
        assert np.abs(got[r0:r1] - run_mean[c - n:]).max() <= 1e-12
    exact = _prefill(orp, case, kc, vc)
    b0 = int(case.block_tables[1][0])
    assert np.array_equal(exact[int(case.query_start[1])], vw[b0, :, 0, :])


PREFILL_PINS = [
    pin_prefill_bruteforce,
    pin_prefill_library,
    pin_prefill_single_query,
    pin_prefill_chunking,
    pin_prefill_closed_forms,
]


def pin_swap(orc):
    """Swapping out to a smaller host pool and back in under new block ids
    restores every block bit for bit; blocks not named keep their bits; and
    decode through the relabelled table equals decode before the swap."""
    case = wl.random_case(24, 3, 2, 8, 4, "bf16", ctx=[7, 13, 4], spare_blocks=9)
    N = case.num_blocks
    held = [sorted(int(b) for b in case.block_tables[s] if b >= 0) for s in range(case.num_seqs)]
    # Preempt sequence 1: its blocks go to host slots 0.. in table order.
    nb1 = -(-int(case.context_lens[1]) // case.block_size)
    out_ids = [int(case.block_tables[1, j]) for j in range(nb1)]
    host_k = wl.canary_fill((nb1 + 2,) + case.k_cache.shape[1:], "bf16")
    host_v = wl.canary_fill((nb1 + 2,) + case.v_cache.shape[1:], "bf16")
    out_pairs = np.array([[b, i + 1] for i, b in enumerate(out_ids)], dtype=np.int64)
    hk, hv = orc.swap_blocks(case.k_cache, case.v_cache, host_k, host_v, out_pairs)
    for i, b in enumerate(out_ids):
        assert np.array_equal(hk[i + 1].view(np.uint16), case.k_cache[b].view(np.uint16))
        assert np.array_equal(hv[i + 1].view(np.uint16), case.v_cache[b].view(np.uint16))
    for i in (0, nb1 + 1):  # host slots not named keep their canaries
        assert np.array_equal(hk[i].view(np.uint16), host_k[i].view(np.uint16))
    # Resume: swap back into free device blocks (ids not used by any sequence).
    used = {b for h in held for b in h}
    free = [b for b in range(N) if b not in used][:nb1]
    in_pairs = np.array([[i + 1, f] for i, f in enumerate(free)], dtype=np.int64)
    kc2, vc2 = orc.swap_blocks(hk, hv, case.k_cache, case.v_cache, in_pairs)
    for i, f in enumerate(free):
        assert np.array_equal(kc2[f].view(np.uint16), case.k_cache[out_ids[i]].view(np.uint16))
    keep = [b for b in range(N) if b not in free]
    assert np.array_equal(kc2[keep].view(np.uint16), case.k_cache[keep].view(np.uint16))
    bt = case.block_tables.copy()
    bt[1, :nb1] = free
    got = orc.paged_decode(case.q, kc2, vc2, bt, case.context_lens, case.scale, case.dtype)
    ref = brute_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, case.scale,
                       case.dtype)
    assert np.abs(got - ref).max() <= 1e-12


ALL_PINS.append(pin_swap)


# ---------------------------------------------------------------------------
# Block manager model pins (take the oracle.block_manager module)
# ---------------------------------------------------------------------------


def _bm_check_invariants(bm, B):
    """Reference counts equal table references; free, evictable and held
    blocks partition the pool; every table holds ceil(len / B) blocks; every
    cached block is full and holds the tokens its key names."""
    refs = [0] * bm.num_blocks
    for s, t in bm.tables.items():
        assert len(t) == -(-bm.lens[s] // B), (s, len(t), bm.lens[s])
        for b in t:
            refs[b] += 1
    assert refs == bm.ref
    free, ev = set(bm.free), set(bm.evictable)
    held = {b for b in range(bm.num_blocks) if bm.ref[b] > 0}
    assert len(free) == len(bm.free) and not (free & ev) and not (free & held) and not (ev & held)
    assert free | ev | held == set(range(bm.num_blocks))
    for key, b in bm.cache.items():
        assert bm.key_of[b] == key and len(key[1]) == B


def pin_bm_digest_flowchart(obm):
    """The digest's flowchart: with B = 16 and blocks handed out as P3, P7,
    P1, P5, P9, sequence 1 (33 tokens) gets P3, P7, P1; sequence 2, whose
    prompt shares sequence 1's first 16 tokens, reuses the shared P3 and gets
    P5 for its 17th token.  A write into a shared, partly filled block copies
    it first (writer takes the copy): P3 -> P9 in a pool where P9 is next."""
    g = _golden("digest_flowchart_layout.json")
    B, N = g["block_size"], g["pool_blocks"]
    order = [3, 7, 1, 5, 9] + [b for b in range(N) if b not in (3, 7, 1, 5, 9)]
    bm = obm.BlockManagerModel(N, B, order, prefix_cache=True)
    p1 = list(range(100, 133))
    assert bm.add_seq(1, p1) == 0
    bm.append(1, 33, p1)
    p2 = p1[:16] + [999]
    assert bm.add_seq(2, p2) == 16
    bm.append(2, 1, p2[16:])
    assert bm.table(1) == g["tables"]["seq1"] and bm.table(2) == g["tables"]["seq2"]
    assert bm.ref[g["shared_block"]] == 2
    _bm_check_invariants(bm, B)
    cow = obm.BlockManagerModel(N, B, [g["cow"]["src"], g["cow"]["dst"]] +
                                [b for b in range(N) if b not in (g["cow"]["src"], g["cow"]["dst"])])
    cow.add_seq(1)
    cow.append(1, 10)
    cow.fork(1, 2)
    slots, pairs = cow.append(2, 1)
    assert pairs == [(g["cow"]["src"], g["cow"]["dst"])]
    assert cow.table(2) == [g["cow"]["dst"]] and cow.table(1) == [g["cow"]["src"]]
    assert slots == [g["cow"]["dst"] * B + 10] and cow.ref[g["cow"]["src"]] == 1
    _bm_check_invariants(cow, B)


def pin_bm_matches_harness(obm):
    """Random append / fork / free traces give the same tables, slots and
    copy pairs as the input generators' own allocator (written separately)."""
    from workloads.blockpool import BlockPool, SeqBlocks, append_tokens, fork

    for seed in range(6):
        rng = np.random.default_rng(300 + seed)
        N, B = 96, int(rng.choice([1, 2, 4, 8]))
        order = rng.permutation(N)
        bm = obm.BlockManagerModel(N, B, order)
        pool = BlockPool(N, B, order)
        live = {}  # seq id -> harness SeqBlocks
        nxt = 0
        for _ in range(60):
            op = rng.integers(0, 4)
            if op == 0 or not live:
                n = int(rng.integers(0, 3 * B + 2))
                if pool.used * 1.0 + n / B + 2 > N * 0.6:
                    continue
                live[nxt] = SeqBlocks()
                bm.add_seq(nxt)
                sl_h, pr_h = append_tokens(pool, live[nxt], n)
                sl_m, pr_m = bm.append(nxt, n)
                assert (sl_h, pr_h) == (sl_m, pr_m)
                nxt += 1
            elif op == 1:
                s = int(rng.choice(list(live)))
                n = int(rng.integers(1, B + 2))
                if pool.used + n // B + 2 > N * 0.8:
                    continue
                sl_h, pr_h = append_tokens(pool, live[s], n)
                sl_m, pr_m = bm.append(s, n)
                assert (sl_h, [tuple(p) for p in pr_h]) == (sl_m, pr_m)
            elif op == 2:
                s = int(rng.choice(list(live)))
                k = int(rng.integers(1, 4))
                kids = fork(pool, live.pop(s), k)
                for kid in kids:
                    bm.fork(s, nxt)
                    live[nxt] = kid
                    nxt += 1
                bm.free_seq(s)
            else:
                s = int(rng.choice(list(live)))
                for b in live.pop(s).table:
                    pool.release(b)
                bm.free_seq(s)
            for s, sb in live.items():
                assert bm.table(s) == sb.table and bm.length(s) == sb.length
            assert list(bm.free) == list(pool.free)
            _bm_check_invariants(bm, B)


def pin_bm_prefix_cache(obm):
    """Hand-derived prefix-cache scenario (B = 4, blocks handed out 0, 1, 2, ...)."""
    bm = obm.BlockManagerModel(12, 4, prefix_cache=True)
    A = list(range(1, 11))                       # 10 tokens: blocks 0, 1 full, 2 partial
    assert bm.add_seq(0, A) == 0
    bm.append(0, 10, A)
    assert bm.table(0) == [0, 1, 2]
    Bp = list(range(1, 9)) + [50, 51]            # shares A's first two blocks
    assert bm.add_seq(1, Bp) == 8
    bm.append(1, 2, Bp[8:])
    assert bm.table(1) == [0, 1, 3] and bm.ref[0] == 2 and bm.ref[1] == 2
    C = [1, 2, 3, 4, 99, 98, 97, 96, 95]         # shares one block only
    assert bm.add_seq(2, C) == 4
    bm.append(2, 5, C[4:])
    assert bm.table(2) == [0, 4, 5]
    D = list(range(1, 9))                        # exactly two cached blocks: reuse one, compute the rest
    assert bm.add_seq(3, D) == 4
    bm.append(3, 4, D[4:])
    assert bm.table(3) == [0, 6]                 # block 6 now duplicates block 1's content, uncached
    Wrong = [9, 9, 9, 9, 5, 6, 7, 8, 1]          # second block matches A's tokens but the prefix differs
    assert bm.add_seq(4, Wrong) == 0
    # Sequence 3's block 6 duplicates cached block 1, so it is not the cached
    # one; a block filled after it is still identified by the whole prefix:
    # extend sequence 3 by one block and look it up from a fresh prompt.
    bm.append(3, 4, [20, 21, 22, 23])             # block 7 = prefix 1..8 + 20..23
    assert bm.table(3) == [0, 6, 7]
    F = list(range(1, 9)) + [20, 21, 22, 23, 0]
    assert bm.add_seq(7, F) == 12 and bm.table(7) == [0, 1, 7]
    bm.free_seq(7)
    G = [5, 5, 5, 5, 5, 5, 5, 5, 20, 21, 22, 23, 0]  # same third block, different prefix: no hit past it
    assert bm.add_seq(8, G) == 0
    bm.free_seq(8)
    for s in (0, 1, 2, 3, 4):
        bm.free_seq(s)
    _bm_check_invariants(bm, 4)
    # Cached blocks survive their sequences and are reused from the evictable set.
    E = list(range(1, 9)) + [7]
    assert bm.add_seq(5, E) == 8
    assert bm.table(5) == [0, 1] and bm.ref[0] == 1 and 0 not in bm.evictable
    # Pool pressure: plain free blocks first, then the least recently released cached block.
    plain = len(bm.free)
    bm.add_seq(6)
    bm.append(6, 4 * plain, list(range(1000, 1000 + 4 * plain)))  # uses every plain free block
    assert not bm.free
    lru = next(iter(bm.evictable))
    key = bm.key_of[lru]
    bm.append(6, 1, [2000])
    assert bm.table(6)[-1] == lru and key not in bm.cache and lru not in bm.key_of
    _bm_check_invariants(bm, 4)


def pin_bm_out_of_blocks(obm):
    """An append needing more blocks than are free changes nothing; one
    needing exactly the free blocks succeeds."""
    bm = obm.BlockManagerModel(5, 4)
    bm.add_seq(0)
    bm.append(0, 6)                              # 2 blocks, last partly filled
    bm.fork(0, 1)
    need = bm.blocks_needed(1, 1 + 4 * 3)        # copy of the shared last block + 3 new
    assert need == 4 and bm.num_free() == 3
    snap = (list(bm.free), list(bm.ref), bm.table(0), bm.table(1), bm.length(1))
    try:
        bm.append(1, 1 + 4 * 3)
        raise AssertionError("append beyond the pool succeeded")
    except obm.OutOfBlocks:
        pass
    assert snap == (list(bm.free), list(bm.ref), bm.table(0), bm.table(1), bm.length(1))
    slots, pairs = bm.append(1, 1 + 4 * 2)       # exactly 3 blocks
    assert len(pairs) == 1 and bm.num_free() == 0
    _bm_check_invariants(bm, 4)


def pin_bm_swap(obm):
    """Swapping a sequence out and back in, with the data moved by the
    oracle's swap_blocks along the returned pairs, leaves its decode
    unchanged; the host pool is empty again afterwards."""
    import oracle

    rng = np.random.default_rng(33)
    N, B, H, D = 12, 4, 2, 8
    gpu = obm.BlockManagerModel(N, B, rng.permutation(N))
    host = obm.BlockManagerModel(6, B)
    for s, n in ((0, 7), (1, 9)):
        gpu.add_seq(s)
        gpu.append(s, n)
    kc = wl.canary_fill((N, H, B, D), "f32")
    vc = wl.canary_fill((N, H, B, D), "f32")
    for s in (0, 1):
        for t in range(gpu.length(s)):
            b = gpu.table(s)[t // B]
            kc[b, :, t % B, :] = rng.standard_normal((H, D))
            vc[b, :, t % B, :] = rng.standard_normal((H, D))
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    rows, lens = gpu.block_tables([0, 1], 4)
    before = oracle.paged_decode(q, kc, vc, np.array(rows, np.int32), np.array(lens, np.int32), 0.3, "f32")
    hk = wl.canary_fill((6, H, B, D), "f32")
    hv = wl.canary_fill((6, H, B, D), "f32")
    out_pairs = gpu.swap_out(1, host)
    assert [p[0] for p in out_pairs] == rows[1][:3] and 1 not in gpu.tables and host.length(1) == 9
    hk, hv = oracle.swap_blocks(kc, vc, hk, hv, out_pairs)
    gpu.add_seq(2)
    gpu.append(2, 9)                             # reuses the freed device blocks
    in_pairs = gpu.swap_in(1, host)
    assert host.num_free() == 6 and gpu.length(1) == 9
    kc, vc = oracle.swap_blocks(hk, hv, kc, vc, in_pairs)
    rows2, lens2 = gpu.block_tables([0, 1], 4)
    after = oracle.paged_decode(q, kc, vc, np.array(rows2, np.int32), np.array(lens2, np.int32), 0.3, "f32")
    assert np.array_equal(before, after)
    _bm_check_invariants(gpu, B)
    _bm_check_invariants(host, B)


BM_PINS = [
    pin_bm_digest_flowchart,
    pin_bm_matches_harness,
    pin_bm_prefix_cache,
    pin_bm_out_of_blocks,
    pin_bm_swap,
]
