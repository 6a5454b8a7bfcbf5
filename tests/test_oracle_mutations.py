"""Planted mistakes in the oracle are caught by the pins.

Each mutant replaces one oracle function (on the CPU, inside this process
only) with a plausible wrong version: a dropped term, a flipped sign, a
wrong index or a transposed operand.  The test passes only if at least one
pin of ``oracle_pins.ALL_PINS`` rejects the mutant, which shows the pins are
strong enough to catch that class of mistake in the real oracle.
"""
import numpy as np
import pytest

import oracle.paged_attention as opa
from oracle_pins import ALL_PINS

_real = {name: getattr(opa, name) for name in dir(opa) if not name.startswith("_")}


def _attention_no_scale(q, K, V, scale):
    return _real["attention"](q, K, V, 1.0)


def _attention_flipped(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s.max() - s)
    return (w / w.sum()) @ V


def _attention_unnormalised(q, K, V, scale):
    s = scale * (K @ q)
    return np.exp(s - s.max()) @ V


def _attention_weights_on_k(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ K


def _logical_kv_no_transpose(cache, table_row, ctx):
    _, H, B, D = cache.shape
    nb = _real["blocks_held"](ctx, B)
    blocks = cache[np.asarray(table_row[:nb], dtype=np.int64)]
    return blocks.reshape(H, nb * B, D)[:, :ctx, :] if nb else blocks.reshape(H, 0, D)


def _logical_kv_reversed(cache, table_row, ctx):
    _, H, B, D = cache.shape
    nb = _real["blocks_held"](ctx, B)
    rev = np.asarray(table_row[:nb])[::-1]
    return _real["logical_kv"](cache, np.concatenate([rev, table_row[nb:]]), ctx)


def _logical_kv_drop_last(cache, table_row, ctx):
    full = _real["logical_kv"](cache, table_row, ctx)
    return full[:, : max(1, ctx - 1), :]


def _blocks_floor(n, B):
    return int(n) // int(B)


def _widen_bf16_wrong(a, dtype):
    if dtype == "bf16":
        return (np.asarray(a).astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
    return _real["widen"](a, dtype)


def _reshape_swapped(key, value, k_cache, v_cache, slot_mapping):
    kc, vc = k_cache.copy(), v_cache.copy()
    B = kc.shape[2]
    for i, slot in enumerate(slot_mapping):
        if slot < 0:
            continue
        off, b = divmod(int(slot), B)
        if off < B and b < kc.shape[0]:
            kc[b, :, off, :] = key[i]
            vc[b, :, off, :] = value[i]
    return kc, vc


def _copy_k_only(k_cache, v_cache, pairs):
    kc, _ = _real["copy_blocks"](k_cache, v_cache, pairs)
    return kc, v_cache.copy()


def _merge_no_rescale(parts):
    return sum(o for _, _, o in parts) / sum(l for _, l, _ in parts)


def _decode_wrong_head(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    out = _real["paged_decode"](q, k_cache, v_cache, block_tables, context_lens, scale, dtype)
    return out[:, ::-1, :].copy()


def _partial_no_max(q, K, V, scale):
    s = scale * (K @ q)
    w = np.exp(s - s.min())
    return s.max(), w.sum(), w @ V


def _newest_off_by_one(block_tables, context_lens, block_size):
    return _real["newest_token_slots"](block_tables, np.asarray(context_lens) + 1, block_size)


def _decode_gqa_modulo(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Query head h reads K/V head h % Hk instead of h // G."""
    H, Hk = q.shape[1], k_cache.shape[1]
    perm = np.array([(h % Hk) * (H // Hk) + h // Hk for h in range(H)]) if H != Hk else np.arange(H)
    out = _real["paged_decode"](q[:, perm], k_cache, v_cache, block_tables, context_lens, scale, dtype)
    inv = np.argsort(perm)
    return out[:, inv]


def _swap_k_only(src_k, src_v, dst_k, dst_v, pairs):
    kd, _ = _real["swap_blocks"](src_k, src_v, dst_k, dst_v, pairs)
    return kd, dst_v.copy()


def _swap_reversed_pairs(src_k, src_v, dst_k, dst_v, pairs):
    """(dst, src) read as (src, dst)."""
    pr = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)[:, ::-1]
    return _real["swap_blocks"](src_k, src_v, dst_k, dst_v, np.ascontiguousarray(pr))


MUTANTS = {
    "attention drops the scale": ("attention", _attention_no_scale),
    "softmax exponent sign flipped": ("attention", _attention_flipped),
    "softmax not normalised": ("attention", _attention_unnormalised),
    "weights applied to K instead of V": ("attention", _attention_weights_on_k),
    "block layout not transposed": ("logical_kv", _logical_kv_no_transpose),
    "block table walked backwards": ("logical_kv", _logical_kv_reversed),
    "last context token dropped": ("logical_kv", _logical_kv_drop_last),
    "blocks held rounds down": ("blocks_held", _blocks_floor),
    "bf16 widened with the wrong shift": ("widen", _widen_bf16_wrong),
    "slot split into (offset, block)": ("reshape_and_cache", _reshape_swapped),
    "block copy skips V": ("copy_blocks", _copy_k_only),
    "partials merged without rescaling": ("merge_partials", _merge_no_rescale),
    "heads transposed in the output": ("paged_decode", _decode_wrong_head),
    "partial stats use the wrong reference": ("partial_attention", _partial_no_max),
    "newest token taken one position late": ("newest_token_slots", _newest_off_by_one),
    "query heads grouped round-robin over K/V heads": ("paged_decode", _decode_gqa_modulo),
    "swap moves K only": ("swap_blocks", _swap_k_only),
    "swap pairs read backwards": ("swap_blocks", _swap_reversed_pairs),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(opa, attr, fn)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(opa)
        except Exception as e:  # a pin rejecting the mutant, by assertion or otherwise
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake: {name}"


# ---------------------------------------------------------------------------
# Prefill oracle mutants (checked against oracle_pins.PREFILL_PINS)
# ---------------------------------------------------------------------------

import oracle.prefill as opr  # noqa: E402
from oracle_pins import PREFILL_PINS  # noqa: E402

_real_pf = {name: getattr(opr, name) for name in ("causal_rows", "paged_prefill")}


def _rows_no_diagonal(Q, K, V, scale, first_pos):
    """Each query attends to the keys strictly before it (its own key missing)."""
    out = np.empty((Q.shape[0], Q.shape[1]))
    for i in range(Q.shape[0]):
        p = first_pos + i
        m = max(p, 1)
        out[i] = opa.attention(Q[i], K[:m], V[:m], scale)
    return out


def _rows_unmasked(Q, K, V, scale, first_pos):
    """Every query attends to the whole context (no causal mask)."""
    return np.stack([opa.attention(Q[i], K, V, scale) for i in range(Q.shape[0])])


def _rows_top_left(Q, K, V, scale, first_pos):
    """The chunk placed at the start of the context instead of its end."""
    return _real_pf["causal_rows"](Q, K, V, scale, 0)


def _rows_one_early(Q, K, V, scale, first_pos):
    """The chunk placed one position early (each query misses its own key
    once a prefix exists)."""
    return _real_pf["causal_rows"](Q, K, V, scale, max(first_pos - 1, 0))


def _prefill_fixed_stride(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype):
    """Packed rows read as if every sequence's chunk had the longest length."""
    qs = np.asarray(query_start)
    n_max = int(np.diff(qs).max())
    fake = np.minimum(np.arange(len(qs)) * n_max, qs[-1])
    fake = np.maximum.accumulate(np.minimum(fake, qs[-1]))
    fake[-1] = qs[-1]
    return _real_pf["paged_prefill"](q, k_cache, v_cache, block_tables, context_lens, fake, scale, dtype)


def _prefill_gqa_modulo(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype):
    """Query head h reads K/V head h % Hk instead of h // G."""
    H, Hk = q.shape[1], k_cache.shape[1]
    perm = np.array([(h % Hk) * (H // Hk) + h // Hk for h in range(H)]) if H != Hk else np.arange(H)
    out = _real_pf["paged_prefill"](q[:, perm], k_cache, v_cache, block_tables, context_lens, query_start, scale,
                                    dtype)
    return out[:, np.argsort(perm)]


PREFILL_MUTANTS = {
    "causal mask drops the diagonal": ("causal_rows", _rows_no_diagonal),
    "no causal mask": ("causal_rows", _rows_unmasked),
    "chunk aligned to the start of the context": ("causal_rows", _rows_top_left),
    "chunk placed one position early": ("causal_rows", _rows_one_early),
    "packed rows read with a fixed stride": ("paged_prefill", _prefill_fixed_stride),
    "prefill heads grouped round-robin over K/V heads": ("paged_prefill", _prefill_gqa_modulo),
}


@pytest.mark.parametrize("name", list(PREFILL_MUTANTS))
def test_prefill_mutant_is_caught(name, monkeypatch):
    attr, fn = PREFILL_MUTANTS[name]
    monkeypatch.setattr(opr, attr, fn)
    failures = []
    for pin in PREFILL_PINS:
        try:
            pin(opr)
        except Exception as e:
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake: {name}"


# ---------------------------------------------------------------------------
# Block manager model mutants (checked against oracle_pins.BM_PINS)
# ---------------------------------------------------------------------------

import oracle.block_manager as obm  # noqa: E402
from oracle_pins import BM_PINS  # noqa: E402

_BMM = obm.BlockManagerModel
_real_bm = {n: getattr(_BMM, n) for n in ("_allocate", "_release", "append", "add_seq", "_block_key", "swap_out")}


def _bm_alloc_lifo(self):
    if self.free:
        self.free.rotate(1)  # take the most recently freed block instead of the oldest
    return _real_bm["_allocate"](self)


def _bm_release_leaks(self, b):
    self.ref[b] -= 1  # never returns to the free list


def _bm_append_no_cow(self, seq, n, tokens=None):
    saved = self.ref
    self.ref = _NoShare(saved)
    try:
        return _real_bm["append"](self, seq, n, tokens)
    finally:
        self.ref = saved


class _NoShare(list):
    """Reference counts that read as 1 for the write path (no copy-on-write)."""

    def __init__(self, base):
        super().__init__(base)
        self.base = base

    def __getitem__(self, i):
        v = self.base[i]
        return min(v, 1) if isinstance(i, int) else v

    def __setitem__(self, i, v):
        self.base[i] = v
        super().__setitem__(i, v)


def _bm_add_whole_prompt(self, seq, prompt=None):
    """Prefix reuse may cover the entire prompt (nothing left to compute)."""
    if prompt:
        prompt = list(prompt) + [object()]  # one phantom token: the last real block becomes reusable
    n = _real_bm["add_seq"](self, seq, prompt)
    self.tokens[seq] = [t for t in self.tokens[seq] if not isinstance(t, object) or isinstance(t, int)]
    return n


def _bm_key_no_prefix(self, seq, j):
    return ((), tuple(self.tokens[seq][j * self.B:(j + 1) * self.B]))


def _bm_swap_reversed(self, seq, host):
    """Pairs send the device blocks to the host blocks in reverse order while
    the host table keeps the allocation order (data and table disagree)."""
    pairs = _real_bm["swap_out"](self, seq, host)
    hosts = [h for _, h in pairs][::-1]
    return [(d, h) for (d, _), h in zip(pairs, hosts)]


def _bm_append_unchecked(self, seq, n, tokens=None):
    self.num_free = lambda: 1 << 30  # skips the up-front capacity check
    try:
        return _real_bm["append"](self, seq, n, tokens)
    except obm.OutOfBlocks:
        raise
    finally:
        del self.num_free


BM_MUTANTS = {
    "free list taken last-in first-out": ("_allocate", _bm_alloc_lifo),
    "released blocks never freed": ("_release", _bm_release_leaks),
    "no copy-on-write of a shared block": ("append", _bm_append_no_cow),
    "prefix reuse covers the whole prompt": ("add_seq", _bm_add_whole_prompt),
    "prefix identity ignores the blocks before": ("_block_key", _bm_key_no_prefix),
    "swap-out pairs disagree with the host table": ("swap_out", _bm_swap_reversed),
    "append without the capacity check": ("append", _bm_append_unchecked),
}


@pytest.mark.parametrize("name", list(BM_MUTANTS))
def test_block_manager_mutant_is_caught(name, monkeypatch):
    attr, fn = BM_MUTANTS[name]
    monkeypatch.setattr(_BMM, attr, fn)
    failures = []
    for pin in BM_PINS:
        try:
            pin(obm)
        except Exception as e:
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin caught the planted mistake: {name}"
