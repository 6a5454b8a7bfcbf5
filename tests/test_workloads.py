"""Input generators: seeded, well-formed, and honest about their canaries."""
import math

import numpy as np
import pytest
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10, np.float32([0.0, -0.0, 1e-40, 3.0e38, 1 + 2**-8, 1 + 3 * 2**-8])])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.float16).numpy()
    assert np.array_equal(wl.to_storage(x, "f16").view(np.uint16), ref.view(np.uint16))


def test_rng_is_thread_count_independent(monkeypatch):
    import workloads.rng as r

    a = r.normal_f32(5, "t", 3 * r.CHUNK + 17)
    monkeypatch.setattr(r, "_threads", lambda: 1)
    b = r.normal_f32(5, "t", 3 * r.CHUNK + 17)
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 1e-3 and abs(a.std() - 1) < 1e-3


def _check_case(case: wl.Case):
    S = case.num_seqs
    B, N = case.block_size, case.num_blocks
    seen = set()
    for s in range(S):
        n = int(case.context_lens[s])
        nb = math.ceil(n / B)
        row = case.block_tables[s]
        assert (row[:nb] >= 0).all() and (row[:nb] < N).all()
        assert (row[nb:] == -1).all()
        blocks = set(row[:nb].tolist())
        assert len(blocks) == nb
        seen |= blocks
    return seen


@pytest.mark.parametrize("make", [wl.tiny_f32, wl.llama7b_decode, wl.opt13b_decode],
                         ids=["tiny-f32", "llama7b", "opt13b"])
def test_block_tables_are_well_formed(make):
    case = make()
    used = _check_case(case)
    # No two sequences share a block in workloads without forking.
    assert len(used) == sum(math.ceil(int(c) / case.block_size) for c in case.context_lens)
    # Every slot outside the valid tokens holds the canary; valid slots do not.
    bits = wl.bits_view(case.k_cache)
    canary = wl.CANARY_BITS[case.dtype]
    valid = np.zeros(case.k_cache.shape[:1] + case.k_cache.shape[2:3], dtype=bool)
    n_append = 1 if case.steps else 0
    for s in range(case.num_seqs):
        for t in range(int(case.context_lens[s]) - n_append):
            valid[case.block_tables[s, t // case.block_size], t % case.block_size] = True
    per_slot = bits.transpose(0, 2, 1, 3)
    assert (per_slot[~valid] == canary).all()
    assert (per_slot[valid] != canary).all()


def test_tiny_f32_shape():
    c = wl.tiny_f32()
    assert c.context_lens.tolist() == [5, 16, 37]
    assert c.num_blocks == 16 and c.meta["blocks_used"] == 16
    assert c.q.dtype == np.float32 and c.scale == pytest.approx(1 / math.sqrt(8))


def test_opt13b_append_slots():
    c = wl.opt13b_decode()
    st = c.steps[0]
    assert st.key.shape == (256, 40, 128)
    assert np.unique(st.slot_mapping).size == 256
    for s in range(256):
        t = int(c.context_lens[s]) - 1
        assert st.slot_mapping[s] == c.block_tables[s, t // 16] * 16 + t % 16
    assert c.context_lens.min() >= 16 and c.context_lens.max() <= 2048


@pytest.mark.parametrize("B", [8, 16, 32])
def test_parallel_sampling_cow_structure(B):
    c = wl.parallel_sampling(block_size=B, num_prompts=8, num_heads=2, head_dim=8, pool_tokens=65536)
    ap0, cp, ap1 = c.steps
    assert cp.pairs.shape == (8 * 3, 2)
    src, dst = cp.pairs[:, 0], cp.pairs[:, 1]
    assert np.unique(dst).size == dst.size and not np.intersect1d(src, dst).size
    last = math.ceil(500 / B) - 1
    for g in range(8):
        rows = c.block_tables[4 * g : 4 * g + 4]
        # Full prompt blocks are shared by all four samples.
        assert (rows[:, :last] == rows[0, :last]).all()
        # Samples 0..2 own copies of the partial last block; sample 3 keeps it.
        assert len(set(rows[:, last].tolist())) == 4
        for i in range(3):
            assert (rows[i, last], ) in {(d,) for d in dst}
            assert [rows[3, last], rows[i, last]] in cp.pairs.tolist()
    allslots = np.concatenate([ap0.slot_mapping, ap1.slot_mapping])
    assert np.unique(allslots).size == allslots.size
    assert 0.5 < c.meta["kv_memory_saved"] < 0.65


def test_random_case_ctx_zero_and_padding():
    c = wl.random_case(3, 3, 2, 8, 4, "f16", ctx=[0, 1, 9])
    assert (c.block_tables[0] == -1).all()
    _check_case(c)


@pytest.mark.parametrize("kind", ["llama7b", "llama3-8b", "prompts"])
def test_prefill_config_structure(kind):
    case = wl.prefill_config(kind)
    qs = case.query_start
    n = np.diff(qs)
    assert qs[0] == 0 and qs[-1] == case.num_tokens == case.q.shape[0]
    assert (n >= 1).all() and (n <= case.context_lens).all()
    st = case.steps[0]
    assert st.slot_mapping.size == case.num_tokens
    # The chunk's slots are the positions ctx - n .. ctx - 1 of each sequence, in order.
    B = case.block_size
    r = 0
    for s in range(case.num_seqs):
        c = int(case.context_lens[s])
        for pos in range(c - int(n[s]), c):
            slot = int(st.slot_mapping[r])
            assert slot == int(case.block_tables[s, pos // B]) * B + pos % B
            r += 1
    if kind == "prompts":
        assert (n == case.context_lens).all()  # whole prompts, nothing cached before
    else:
        assert (n == 512).all() and case.num_seqs == 16


def test_random_prefill_case_is_seeded():
    a = wl.random_prefill_case(9, [2, 0], [3, 4], 2, 8, 4, "bf16")
    b = wl.random_prefill_case(9, [2, 0], [3, 4], 2, 8, 4, "bf16")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.k_cache.view(np.uint16), b.k_cache.view(np.uint16))
