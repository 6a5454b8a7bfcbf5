"""Host-side check of the decode kernels' address arithmetic.

Mirrors the index formulas of the vector partition kernel
(``csrc/pa_decode_impl.h``) and of the matrix-core kernel
(``csrc/pa_decode_mfma.h``): launch geometry, partition bounds, LDS staging
of block ids and merge buffers, clamped token addresses, query and workspace
slots, and asserts that, for every workload the GPU tests and the benchmark
launch, every read and write stays inside its buffer.  Runs on the CPU only.
"""
import functools
import math

import numpy as np
import pytest

import workloads as wl

MAX_PART_BLOCKS = 8192


BALANCED_MIN_CHUNK = 256


def balanced_plan(S, Hk, max_ctx, G=1, partition=0):
    """Mirror of plan_decode's choice of the balanced split."""
    pairs = S * Hk
    return G >= 2 and partition == 0 and pairs < 512 and S <= 512 and pairs * max_ctx < (1 << 31)


def default_partition(S, Hk, max_ctx, G=1):
    """Mirror of the library's default partition rule (plan_decode): the
    partition length, or under a balanced plan its smallest share."""
    if balanced_plan(S, Hk, max_ctx, G):
        return BALANCED_MIN_CHUNK
    pmin, lpt = (512, 512) if G >= 2 else (256, 1024)
    whole = pmin
    while whole < 4096 and whole < max_ctx:
        whole *= 2
    if S * Hk >= 8192 or (S * Hk >= lpt and S <= 512):
        return whole
    part = whole
    while part > pmin and S * Hk * (-(-max_ctx // part)) < 8192:
        part //= 2
    return part


def shape(elem, D, G=1):
    vec = 16 // elem
    lpr = D // vec
    tpl = 64 // lpr
    nl = max(1, min(8, (16 if G <= 2 else 8) // tpl))
    return vec, lpr, tpl, nl, nl * tpl


def check_decode_bounds(S, H, D, B, N, W, elem, ctx, bt, max_ctx, part, G=1):
    """H is the caches' head count (K/V heads); G query heads share each."""
    vec, lpr, tpl, nl, U = shape(elem, D, G)
    staged = (part + B - 1) // B + 1
    assert staged <= MAX_PART_BLOCKS  # host check in pa_decode; LDS holds `staged` ids
    assert max_ctx <= W * B  # host check in pa_decode
    log2b = B.bit_length() - 1
    assert 1 << log2b == B
    max_parts = max(1, math.ceil(max_ctx / part))
    cache_elems = N * H * B * D
    blk_stride = H * B * D
    head_off_max = (H - 1) * B * D + (lpr - 1) * vec
    ws_o_elems = S * H * max_parts * D
    for s in range(S):
        c = int(ctx[s])
        for p in range(max_parts):
            if c <= 0 or c > max_ctx:
                continue  # writes out[s, h, :] only
            t_begin = p * part
            if t_begin >= c:
                continue
            t_end = min(c, t_begin + part)
            j0 = t_begin >> log2b
            nblk = ((t_end - 1) >> log2b) - j0 + 1
            assert 1 <= nblk <= staged
            assert 0 <= j0 and j0 + nblk - 1 < W  # block-table row reads
            niter = (t_end - t_begin + U - 1) // U
            # K/V head hk walks the steps from hk * niter // H on, wrapping
            # around: every step exactly once, whatever the head.
            for hk in {0, H // 2, H - 1}:
                order = (np.arange(niter) + hk * niter // H) % niter
                assert np.array_equal(np.sort(order), np.arange(niter))
            ts = np.arange(niter)[:, None, None] * U + np.arange(nl)[None, :, None] * tpl + np.arange(tpl)[None, None, :]
            t = np.minimum(t_begin + ts, t_end - 1).ravel()
            assert t.min() >= t_begin
            lds = (t >> log2b) - j0
            assert lds.min() >= 0 and lds.max() < nblk
            b = bt[s, j0 + lds]
            b = np.where((b >= 0) & (b < N), b, 0)  # invalid ids are flagged and replaced by 0
            e = b.astype(np.int64) * blk_stride + (t & (B - 1)).astype(np.int64) * D
            assert e.min() >= 0 and e.max() + head_off_max + vec <= cache_elems
            if c > part:  # workspace rows are per query head: S * H * G of them
                assert ((s * H * G + H * G - 1) * max_parts + p) * D + D <= ws_o_elems * G


MFMA_TILE = 16
MFMA_WAVES = 8
MFMA_MERGE_FLOATS = 8192


def mfma_merge_heads(D, G):
    hc0 = MFMA_MERGE_FLOATS // (MFMA_WAVES * (D + 4))
    for hc in (G, 8, 4, 2, 1):
        if hc <= hc0 or hc == 1:
            return hc


def check_mfma_bounds(S, Hk, G, D, B, N, W, ctx, bt, max_ctx, part):
    """The matrix-core kernel: 16-token tiles; lane (c, g) = (lane % 16, lane // 16)
    reads key channels 32 ks + 8 g .. +7 of token tb + c and value channels
    E c .. E c + E - 1 (E = D / 16) of tokens tb + 4 g + i; the query operand
    is head c < G; merge rows s_o[wave][c - c0][E (4 g + j) + t]."""
    assert D in (64, 128, 256)
    E = D // 16
    KS = D // 32
    c = np.arange(16)
    g = np.arange(4)
    # Per-lane channel extents inside one row of D elements.
    k_lo = (32 * np.arange(KS)[:, None] + 8 * g[None, :]).ravel()
    assert k_lo.min() >= 0 and k_lo.max() + 8 <= D
    v_lo = E * c
    assert v_lo.max() + E <= D
    # Query rows: head sh0 + c for c < G only (the rest are zero operands).
    H = Hk * G
    q_rows = (np.arange(S)[:, None] * H + np.arange(Hk)[None, :] * G)[..., None] + np.arange(G)
    assert q_rows.max() * D + D <= S * H * D
    # Merge buffer indices.
    hc = mfma_merge_heads(D, G)
    assert G % hc == 0
    col = 16 * np.arange(E)[None, None, :] + 4 * g[:, None, None] + np.arange(4)[None, :, None]
    assert col.min() >= 0 and col.max() < D and len(np.unique(col)) == D
    assert MFMA_WAVES * hc * (D + 4) <= MFMA_MERGE_FLOATS or hc == 1
    staged = (part + B - 1) // B + 1
    max_parts = max(1, math.ceil(max_ctx / part))
    for s in range(S):
        cl = int(ctx[s])
        if cl <= 0 or cl > max_ctx:
            continue
        for p in range(max_parts):
            t_begin = p * part
            if t_begin >= cl:
                continue
            mfma_run_checks(s, cl, t_begin, min(cl, t_begin + part), staged, Hk, D, B, N, W, bt)


def mfma_run_checks(s, cl, t_begin, t_end, staged, Hk, D, B, N, W, bt):
    """One run of the matrix-core kernel over tokens [t_begin, t_end) of
    sequence s (context cl): staged block ids; coalesced K/V loads (load i of
    lane L: token row RPI i + L // (D / 8) of the 16-token tile, clamped to
    t_end - 1, 16-byte chunk L % (D / 8)); the wavefront's LDS tiles (16
    rows of D + 16 elements; K operand rows c, channels 32 ks + 8 g .. +7;
    transposing V reads at rows 4 g + c // 4, channels 16 t + 4 (c % 4) .. +3,
    8-byte aligned)."""
    E, KS = D // 16, D // 32
    c, g = np.arange(16), np.arange(4)
    lane = np.arange(64)
    rpi = 64 * 8 // D
    nld = MFMA_TILE // rpi
    ld_row, ld_ch = lane // (D // 8), lane % (D // 8)
    log2b = B.bit_length() - 1
    blk_stride = Hk * B * D
    cache_elems = N * Hk * B * D
    ldw = D + 16
    assert 0 <= t_begin < t_end <= cl
    j0 = t_begin >> log2b
    nblk = ((t_end - 1) >> log2b) - j0 + 1
    assert 1 <= nblk <= staged and j0 + nblk - 1 < W
    ntile = (t_end - t_begin + MFMA_TILE - 1) // MFMA_TILE
    tb = t_begin + np.arange(ntile)[:, None] * MFMA_TILE
    rows = (rpi * np.arange(nld)[:, None] + ld_row[None, :]).ravel()
    assert rows.min() >= 0 and rows.max() < MFMA_TILE and 8 * ld_ch.max() + 8 <= D
    t = np.minimum(tb + rows[None, :], t_end - 1).ravel()
    assert t.min() >= t_begin
    lds = (t >> log2b) - j0
    assert lds.min() >= 0 and lds.max() < nblk
    b = bt[s, j0 + lds]
    b = np.where((b >= 0) & (b < N), b, 0)
    e = b.astype(np.int64) * blk_stride + (Hk - 1) * B * D + (t & (B - 1)).astype(np.int64) * D
    assert e.min() >= 0 and e.max() + 8 * ld_ch.max() + 8 <= cache_elems
    # LDS tile reads and writes stay inside the wavefront's 2 x 16 x ldw tile.
    assert (MFMA_TILE - 1) * ldw + 8 * ld_ch.max() + 8 <= MFMA_TILE * ldw
    k_hi = (MFMA_TILE - 1) * ldw + 32 * (KS - 1) + 8 * 3 + 8
    assert k_hi <= MFMA_TILE * ldw
    tr = (4 * g[:, None] + c[None, :] // 4) * ldw + 4 * (c[None, :] % 4)
    tr_all = tr[..., None] + 16 * np.arange(E)
    assert tr_all.max() + 4 <= MFMA_TILE * ldw and (tr_all % 4 == 0).all() and (ldw * 2) % 8 == 0
    assert (16 * (E - 1) + 4 * 3 + 4) <= D  # a row's channels only
    # The newest token (append) is token cl - 1, covered by the last tile.
    if t_end == cl:
        last = tb[-1, 0]
        assert last <= cl - 1 < last + MFMA_TILE


def check_balanced_bounds(S, Hk, G, D, B, N, W, ctx, bt, max_ctx, num_wgs):
    """The balanced split: each valid (sequence, K/V head) context is cut
    into n = ceil(ctx / C) pieces of ceil(ctx / n) tokens, C = max(256,
    ceil(total / (num_wgs - pairs // 2))); workgroup w (of num_wgs + pairs)
    takes the w-th piece in (sequence, K/V head, piece) order.  Every piece's
    reads stay in bounds, every token is covered exactly once, pieces are
    never empty, the partial slots 0 .. n - 1 match the merge kernel's count
    ceil(ctx / C), and the workspace holds every slot."""
    P = BALANCED_MIN_CHUNK
    max_parts = -(-max_ctx // P) + 1 if max_ctx > 0 else 2
    pairs = S * Hk
    valid = np.array([0 < int(x) <= max_ctx for x in ctx])
    n_tok = np.where(valid, np.asarray(ctx, dtype=np.int64), 0)
    total = Hk * int(n_tok.sum())
    slots = max(1, num_wgs - pairs // 2)
    C = max(P, -(-total // slots))
    assert C < (1 << 31)
    share = min(max(P, -(-(pairs * max_ctx) // slots)), max_ctx)  # host bound of the staged ids
    assert C <= share or C > max_ctx
    staged = -(-share // B) + 1
    pieces = np.where(valid, -(-n_tok // C), 0)
    pre = np.concatenate([[0], np.cumsum(pieces)])
    assert Hk * int(pre[-1]) <= num_wgs + pairs  # the grid covers every piece
    H = Hk * G
    ws_rows = S * H * max_parts
    runs = {}
    for w in range(num_wgs + pairs):
        if w >= Hk * int(pre[-1]):
            continue
        s = int(np.searchsorted(Hk * pre[:S], w, side="right")) - 1
        n = int(pieces[s])
        assert n > 0
        r = w - Hk * int(pre[s])
        hk, slot = r // n, r % n
        cl = int(ctx[s])
        ln = -(-cl // n)
        t0, t1 = slot * ln, min(cl, slot * ln + ln)
        assert t0 < t1 and t1 - t0 <= min(C, share)
        assert slot < max_parts and n == -(-cl // C)  # the merge kernel's count
        mfma_run_checks(s, cl, t0, t1, staged, Hk, D, B, N, W, bt)
        for h in range(hk * G, hk * G + G):
            assert (s * H + h) * max_parts + slot < ws_rows
        runs.setdefault((s, hk), []).append((slot, t0, t1))
    for s in range(S):
        for hk in range(Hk):
            if not valid[s]:
                assert (s, hk) not in runs  # the merge kernel writes 0 or NaN
                continue
            r = sorted(runs[(s, hk)], key=lambda v: v[1])
            assert r[0][1] == 0 and r[-1][2] == int(ctx[s]) and all(a[2] == b[1] for a, b in zip(r, r[1:]))
            assert sorted(v[0] for v in r) == list(range(int(pieces[s])))


CASES = [
    ("tiny-f32", functools.lru_cache(None)(lambda: wl.tiny_f32())),
    ("llama7b-decode", functools.lru_cache(None)(lambda: wl.llama7b_decode())),
    ("opt13b-decode", functools.lru_cache(None)(lambda: wl.opt13b_decode())),
    ("sampling-B8", functools.lru_cache(None)(lambda: wl.parallel_sampling(block_size=8, num_heads=1, head_dim=128))),
    ("sampling-B32", functools.lru_cache(None)(lambda: wl.parallel_sampling(block_size=32, num_heads=1, head_dim=128))),
    ("opt175b-decode", functools.lru_cache(None)(lambda: wl.opt175b_decode(num_heads=2))),
    ("edge", functools.lru_cache(None)(lambda: wl.random_case(21, 5, 2, 64, 1, "bf16", ctx=[0, 1, 2, 513, 700]))),
    ("gqa-llama3-8b", functools.lru_cache(None)(lambda: wl.gqa_config("llama3-8b"))),
    # 12000 short contexts (some empty): tens of thousands of workgroups in batch order
    ("wide-mha", functools.lru_cache(None)(lambda: wl.random_case(92, 12000, 2, 64, 16, "f16", ctx_range=(0, 96)))),
    ("wide-gqa", functools.lru_cache(None)(lambda: wl.random_case(91, 12000, 8, 64, 16, "bf16", ctx_range=(0, 96),
                                                                  num_kv_heads=2))),
    # 128k-token contexts: hundreds of partitions or pieces per context
    ("long-mha", functools.lru_cache(None)(lambda: wl.random_case(93, 4, 4, 128, 16, "f16",
                                                                  ctx=[131072, 70001, 1, 0]))),
    ("long-gqa", functools.lru_cache(None)(lambda: wl.random_case(94, 4, 8, 128, 16, "bf16",
                                                                  ctx=[131072, 70001, 1, 0], num_kv_heads=1))),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("part", [0, 16, 64, 512, 1 << 30])
def test_decode_index_bounds(name, make, part):
    case = make()
    B = case.block_size
    max_ctx = case.max_context_len
    G = case.num_heads // case.num_kv_heads
    p = default_partition(case.num_seqs, case.num_kv_heads, max_ctx, G) if part == 0 else part
    if p == 1 << 30:
        p = max(1, max_ctx)  # a single partition covers every context
    if (p + B - 1) // B + 1 > MAX_PART_BLOCKS:
        pytest.skip("partition rejected by the host check")
    check_decode_bounds(case.num_seqs, case.num_kv_heads, case.head_dim, B, case.num_blocks,
                        case.block_tables.shape[1], case.elem_bytes, case.context_lens,
                        case.block_tables, max_ctx, p, G=case.num_heads // case.num_kv_heads)


def test_invalid_ids_are_clamped_in_the_model():
    """A block id outside the pool is replaced by 0 for the address (and the
    output is flagged NaN), so even garbage tables never address outside the
    caches."""
    case = wl.random_case(22, 2, 1, 8, 4, "f32", ctx=[9, 5])
    bt = case.block_tables.copy()
    bt[0, 1] = 10**6
    bt[1, 0] = -7
    check_decode_bounds(2, 1, 8, 4, case.num_blocks, bt.shape[1], 4, case.context_lens, bt, 9, 4)


MFMA_CASES = [c for c in CASES if c[0] in ("llama7b-decode", "opt13b-decode", "opt175b-decode", "edge", "gqa-llama3-8b",
                                            "sampling-B8", "sampling-B32", "wide-mha", "wide-gqa", "long-mha",
                                            "long-gqa")]


@pytest.mark.parametrize("name,make", MFMA_CASES, ids=[c[0] for c in MFMA_CASES])
@pytest.mark.parametrize("part", [0, 16, 64, 512, 1 << 30])
def test_mfma_index_bounds(name, make, part):
    case = make()
    if case.head_dim not in (64, 128, 256) or case.elem_bytes != 2:
        pytest.skip("matrix-core kernel serves 16-bit caches with D in {64, 128, 256}")
    B = case.block_size
    max_ctx = case.max_context_len
    G = case.num_heads // case.num_kv_heads
    if part == 0 and balanced_plan(case.num_seqs, case.num_kv_heads, max_ctx, G):
        for wgs in (512, 256, 7, 1):
            check_balanced_bounds(case.num_seqs, case.num_kv_heads, G, case.head_dim, B, case.num_blocks,
                                  case.block_tables.shape[1], case.context_lens, case.block_tables, max_ctx, wgs)
        return
    p = default_partition(case.num_seqs, case.num_kv_heads, max_ctx, G) if part == 0 else part
    if p == 1 << 30:
        p = max(1, max_ctx)
    if (p + B - 1) // B + 1 > (4096 if case.head_dim == 256 else 6144):
        pytest.skip("such partitions take the vector kernel")
    check_mfma_bounds(case.num_seqs, case.num_kv_heads, case.num_heads // case.num_kv_heads, case.head_dim, B,
                      case.num_blocks, case.block_tables.shape[1], case.context_lens, case.block_tables, max_ctx, p)


def test_mfma_gqa70b_bounds():
    case = wl.gqa_config("llama2-70b-tp8")
    check_mfma_bounds(case.num_seqs, case.num_kv_heads, 8, case.head_dim, case.block_size, case.num_blocks,
                      case.block_tables.shape[1], case.context_lens, case.block_tables, case.max_context_len, 256)


@pytest.mark.parametrize("wgs", [512, 333, 64])
def test_balanced_gqa70b_bounds(wgs):
    case = wl.gqa_config("llama2-70b-tp8")
    assert balanced_plan(case.num_seqs, case.num_kv_heads, case.max_context_len, 8)
    check_balanced_bounds(case.num_seqs, case.num_kv_heads, 8, case.head_dim, case.block_size, case.num_blocks,
                          case.block_tables.shape[1], case.context_lens, case.block_tables, case.max_context_len, wgs)


@pytest.mark.parametrize("seed", range(6))
def test_balanced_random_lengths(seed):
    """Empty, invalid, tiny and long contexts mixed; shares smaller and
    larger than a context."""
    rng = np.random.default_rng([29, seed])
    S = int(rng.integers(1, 40))
    Hk, G, B = int(rng.choice([1, 2, 4])), int(rng.choice([2, 4, 8])), int(rng.choice([1, 4, 16]))
    ctx = rng.integers(1, 300, S)
    ctx[rng.random(S) < 0.2] = 0
    case = wl.random_case(30 + seed, S, Hk * G, 64, B, "f16", ctx=ctx.tolist(), num_kv_heads=Hk)
    ctx2 = case.context_lens.copy()
    if S > 2:
        ctx2[1] = case.max_context_len + 5  # invalid: skipped, the merge kernel writes NaN
    for wgs in (1, 3, 16, 512):
        check_balanced_bounds(S, Hk, G, 64, B, case.num_blocks, case.block_tables.shape[1], ctx2,
                              case.block_tables, case.max_context_len, wgs)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_mfma_bounds_all_shapes(D, G):
    case = wl.random_case(23, 3, 2 * G, D, 8, "f16", ctx=[1, 37, 300], num_kv_heads=2)
    check_mfma_bounds(3, 2, G, D, 8, case.num_blocks, case.block_tables.shape[1], case.context_lens,
                      case.block_tables, case.max_context_len, 64)


# ---------------------------------------------------------------------------
# Prefill kernel (csrc/pa_prefill.hip)
# ---------------------------------------------------------------------------

PF_ROWS, PF_KEYS, PF_THREADS, PF_MAX_IDS = 128, 32, 256, 4096


def pf_rows(D):
    """Query rows per workgroup: 4 wavefronts x two 16-row blocks, one block at head_dim 256."""
    return PF_ROWS if D <= 128 else PF_ROWS // 2


def check_prefill_bounds(case, max_query_len=None):
    """Grid (H, S, ceil(max_query_len / R)), R = 128 query rows per workgroup
    (64 at head_dim 256); wavefront w of a workgroup owns chunk rows
    r0 + R/4 w + 16 rb + c (rb < R/64); query loads read row min(row, n - 1), channels
    32 ks + 8 g .. +7; block ids of keys 0 .. kv_end - 1 are staged; tile
    loads read key min(kp, kv_end - 1), CPT 16-byte chunks of one row per
    thread (CPR / CPT apart); LDS reads stay in
    the [2][32][D + 16] tiles (K rows 16 sub + c at 32 ks + 8 g .. +7;
    transposing V reads at rows 4 g + c // 4 (+ 16), channels 16 t + 4 (c % 4)
    .. +3, 8-byte aligned); output rows < n, channels 16 t + 4 g .. +3."""
    T, H, D = case.q.shape
    N, Hk, B, _ = case.k_cache.shape
    S = case.num_seqs
    W = case.block_tables.shape[1]
    qs = case.query_start
    n_all = np.diff(qs)
    mq = int(n_all.max()) if max_query_len is None else max_query_len
    assert mq >= n_all.max()
    maxc = case.max_context_len
    ids_cap = -(-maxc // B)
    assert ids_cap <= PF_MAX_IDS and maxc <= W * B
    R = pf_rows(D)
    n_qt = -(-mq // R)
    KS, E, CPR = D // 32, D // 16, D // 8
    assert (PF_KEYS * CPR) % PF_THREADS == 0
    cpt = PF_KEYS * CPR // PF_THREADS
    G = H // Hk
    c = np.arange(16)
    g = np.arange(4)
    # Channel extents inside a row (K operand reads, transposing V reads,
    # output writes), and the 8-byte alignment of the transposing reads.
    LD = D + 16
    assert (32 * (KS - 1) + 8 * g.max() + 8) <= D
    tr_cols = 16 * (E - 1) + 4 * (c % 4)
    assert tr_cols.max() + 4 <= D and (16 + 4 * g.max() + c.max() // 4) < PF_KEYS
    assert (LD * 2) % 8 == 0 and all(((2 * (16 * t + 4 * (c % 4))) % 8 == 0).all() for t in range(E))
    assert 16 * (E - 1) + 4 * g.max() + 4 <= D
    cache_elems = N * Hk * B * D
    for s in range(S):
        n, ctx = int(n_all[s]), int(case.context_lens[s])
        assert 1 <= n <= ctx <= maxc
        for qt in range(n_qt):
            r0 = qt * R
            if r0 >= n:
                continue
            first = ctx - n
            last_row = min(r0 + R, n) - 1
            kv_end = first + last_row + 1
            assert kv_end <= ctx
            nids = ((kv_end - 1) // B) + 1
            assert nids <= ids_cap and nids <= W
            ntiles = -(-kv_end // PF_KEYS)
            # query rows read
            rows = np.minimum(r0 + np.arange(R), n - 1)
            assert int(qs[s]) + rows.max() < T
            # tile loads
            tid = np.arange(PF_THREADS)
            assert CPR % cpt == 0
            ld_row, ld_chunk = tid // (CPR // cpt), tid % (CPR // cpt)
            chunks = [ld_chunk + (CPR // cpt) * u for u in range(cpt)]
            assert ld_row.max() < PF_KEYS and max(ch.max() for ch in chunks) < CPR
            # every (key row, chunk) of a tile is moved exactly once
            assert len({(r, int(ch[i])) for ch in chunks for i, r in enumerate(ld_row)}) == PF_KEYS * CPR
            for kt in range(ntiles):
                kp = np.minimum(kt * PF_KEYS + ld_row, kv_end - 1)  # tail keys re-read the last one
                idx = kp // B
                assert idx.min() >= 0 and idx.max() < nids
                b = case.block_tables[s, idx]
                b = np.where((b >= 0) & (b < N), b, 0).astype(np.int64)
                for u in range(cpt):
                    e = b * Hk * B * D + (Hk - 1) * B * D + (kp % B) * D + 8 * chunks[u]
                    assert e.min() >= 0 and e.max() + 8 <= cache_elems
            # LDS rows read by the compute: keys 16 sub + c and 16 sub + 4 g + j < 32
            assert 16 + 15 < PF_KEYS and 16 + 4 * 3 + 3 < PF_KEYS
        # output rows
        assert int(qs[s]) + n - 1 < T
    assert (H - 1) // G < Hk
    # Every order's linear id -> (sequence, head, query tile) map covers each
    # tile that holds rows exactly once; padding ids exit.
    rows = [prefill_chunk_rows(qs, s, T) for s in range(S)]
    want = {(s_, h, qt) for s_ in range(S) for h in range(H) for qt in range(min(-(-rows[s_] // R), n_qt))}
    for order in ("tile", "unit", "packed"):
        if order != "tile" and S > PF_MAX_RANKED:
            continue
        if order == "packed" and n_qt > PF_MAX_LEVELS:
            continue
        grid = prefill_grid(S, Hk, G, n_qt, T, order, R)
        assert grid <= 0x7FFFFFFF
        got = [w for w in prefill_items(qs, case.context_lens, S, Hk, G, n_qt, T, grid, order, R)]
        got = [w for w in got if w[2] * R < rows[w[0]]]  # tiles past a chunk exit
        assert len(got) == len(set(got)), order
        assert set(got) == want, order


PF_MAX_RANKED, PF_MAX_LEVELS = 64, 64


def prefill_chunk_rows(qs, s, T):
    """Rows of chunk s the kernel serves: 0 when its rows are not inside [0, T)."""
    q0, q1 = int(qs[s]), int(qs[s + 1])
    return q1 - q0 if (q0 >= 0 and q1 > q0 and q1 <= T) else 0


def prefill_order(S, n_qt, T, rows=PF_ROWS):
    """The host's choice of dispatch order (launch_prefill_t)."""
    if S <= PF_MAX_RANKED and 2 * T >= S * n_qt * rows:
        return "unit"
    if S <= PF_MAX_RANKED and n_qt <= PF_MAX_LEVELS:
        return "packed"
    return "tile"


def prefill_grid(S, Hk, G, n_qt, T, order, rows=PF_ROWS):
    padded = -(-(S * Hk) // 8) * 8 * G * n_qt
    if order != "packed":
        return padded
    tiles = (T + (rows - 1) * S) // rows
    per_xcd = -(-(tiles * Hk) // 8) + n_qt
    return min(padded, per_xcd * 8 * G)


def prefill_items(qs, ctx, S, Hk, G, n_qt, T, grid, order, rows=PF_ROWS):
    """(sequence, head, query tile) of every workgroup that does not exit at
    once, as the kernel maps linear ids (XCD = lin % 8 = unit % 8)."""
    units = S * Hk
    if order == "unit":
        rank_to_seq = sorted(range(S), key=lambda i: (-int(ctx[i]), i))
    if order == "packed":
        key = [min(prefill_chunk_rows(qs, i, T), n_qt * rows) for i in range(S)]
        rank_to_seq = sorted(range(S), key=lambda i: (-key[i], i))
        cnt = [sum(k > (n_qt - 1 - j) * rows for k in key) for j in range(n_qt)]  # level j = tile n_qt-1-j
    for lin in range(grid):
        xcd, r8 = lin % 8, lin // 8
        if order == "tile":
            per_tile = grid // (8 * n_qt)
            qt = n_qt - 1 - r8 // per_tile
            unit = ((r8 % per_tile) // G) * 8 + xcd
            if unit >= units:
                continue
            s_, hk, h = unit // Hk, unit % Hk, (unit % Hk) * G + r8 % G
        elif order == "unit":
            per_unit = n_qt * G
            qt = n_qt - 1 - (r8 % per_unit) // G
            unit = (r8 // per_unit) * 8 + xcd
            if unit >= units:
                continue
            s_, hk, h = rank_to_seq[unit // Hk], unit % Hk, (unit % Hk) * G + r8 % G
        else:
            lvl = [(-(-(c * Hk - xcd) // 8)) * G if c * Hk > xcd else 0 for c in cnt]
            base, j = 0, 0
            while j < n_qt and r8 >= base + lvl[j]:
                base += lvl[j]
                j += 1
            if j >= n_qt:
                continue
            off = r8 - base
            unit = (off // G) * 8 + xcd
            assert unit < cnt[j] * Hk  # a unit that has a tile at level j
            s_ = rank_to_seq[unit // Hk]
            hk, h = unit % Hk, (unit % Hk) * G + off % G
            qt = n_qt - 1 - j
            assert qt >= 0 and key[s_] > qt * rows
        assert 0 <= s_ < S and 0 <= h < H_of(Hk, G) and 0 <= qt < n_qt and h // G == hk
        assert unit % 8 == lin % 8  # a unit's workgroups share one XCD
        yield (s_, h, qt)


def H_of(Hk, G):
    return Hk * G


def test_prefill_row_guards_in_the_model():
    """query_start entries that fall, go negative or pass num_tokens leave
    that chunk without rows (skipped); every other chunk's tiles are still
    enumerated by every order, and no served row lies outside [0, T)."""
    T, S, Hk, G = 300, 6, 2, 2
    qs = np.array([0, 50, 40, 120, -5, 200, 400])  # chunk 1 falls, 3 falls, 4 starts below 0, 5 ends past T
    rows = [prefill_chunk_rows(qs, s, T) for s in range(S)]
    assert rows == [50, 0, 80, 0, 0, 0]
    ctx = np.array([60, 10, 80, 90, 200, 500])
    n_qt = 2
    for order in ("tile", "unit", "packed"):
        grid = prefill_grid(S, Hk, G, n_qt, T, order)
        got = {w for w in prefill_items(qs, ctx, S, Hk, G, n_qt, T, grid, order) if w[2] * PF_ROWS < rows[w[0]]}
        assert got == {(s, h, 0) for s in (0, 2) for h in range(Hk * G)}
        for s, _, qt in got:
            assert 0 <= int(qs[s]) and int(qs[s]) + rows[s] <= T


PF_CASES = [
    ("prefill-llama7b", functools.lru_cache(None)(lambda: wl.prefill_config("llama7b"))),
    ("prefill-llama3-8b", functools.lru_cache(None)(lambda: wl.prefill_config("llama3-8b"))),
    ("prefill-prompts", functools.lru_cache(None)(lambda: wl.prefill_config("prompts"))),
    ("prefill-ragged", functools.lru_cache(None)(
        lambda: wl.random_prefill_case(31, [0, 1, 63, 200, 5], [1, 64, 65, 130, 3], 4, 64, 1, "bf16", num_kv_heads=2))),
    # cached prefixes of 60000 and 65000 tokens: up to 4094 staged block ids
    ("prefill-long-f16", functools.lru_cache(None)(
        lambda: wl.random_prefill_case(501, [60000, 0, 3000], [200, 300, 129], 4, 128, 16, "f16", num_kv_heads=2))),
    ("prefill-long-bf16", functools.lru_cache(None)(
        lambda: wl.random_prefill_case(502, [65000, 100], [500, 28], 2, 64, 16, "bf16"))),
    # head_dim 256: 64-row tiles
    ("prefill-d256", functools.lru_cache(None)(
        lambda: wl.random_prefill_case(503, [0, 40, 100], [130, 64, 65], 4, 256, 16, "f16", num_kv_heads=2))),
    ("prefill-d256-prompts", functools.lru_cache(None)(
        lambda: wl.random_prefill_case(504, [200, 0, 0, 3], [1, 200, 333, 64], 8, 256, 8, "bf16"))),
]


@pytest.mark.parametrize("name,make", PF_CASES, ids=[c[0] for c in PF_CASES])
def test_prefill_index_bounds(name, make):
    case = make()
    check_prefill_bounds(case)
    check_prefill_bounds(case, max_query_len=int(np.diff(case.query_start).max()) + 100)


# ---------------------------------------------------------------------------
# The seeded random shapes of tests/test_gpu_random_cases.py, checked here
# before they run on the GPU.
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(48))
def test_random_decode_case_bounds(seed):
    from test_gpu_random_cases import random_decode_case

    case, part = random_decode_case(seed)
    B, D = case.block_size, case.head_dim
    S, Hk = case.num_seqs, case.num_kv_heads
    G = case.num_heads // Hk
    max_ctx = case.max_context_len
    W = case.block_tables.shape[1]
    p = default_partition(S, Hk, max_ctx, G) if part == 0 else part
    assert (p + B - 1) // B + 1 <= MAX_PART_BLOCKS
    check_decode_bounds(S, Hk, D, B, case.num_blocks, W, case.elem_bytes, case.context_lens, case.block_tables,
                        max_ctx, p, G=G)
    if case.elem_bytes == 2 and D in (64, 128, 256) and G >= 2:
        if part == 0 and balanced_plan(S, Hk, max_ctx, G):
            for wgs in (512, 256, 7):
                check_balanced_bounds(S, Hk, G, D, B, case.num_blocks, W, case.context_lens, case.block_tables,
                                      max_ctx, wgs)
        else:
            check_mfma_bounds(S, Hk, G, D, B, case.num_blocks, W, case.context_lens, case.block_tables, max_ctx, p)


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill_case_bounds(seed):
    from test_gpu_random_cases import random_prefill_case

    case = random_prefill_case(seed)
    check_prefill_bounds(case)


# ---------------------------------------------------------------------------
# Sibling-group decode kernel (csrc/pa_decode_siblings.h)
# ---------------------------------------------------------------------------

SIB_MAX, SIB_MAX_IDS, SIB_TILE = 16, 4096, 16


def check_siblings_bounds(case, group, parts=1):
    """Grid (H, ceil(S / group) * ceil(group / sub)), sub = min(group,
    16 // G) members per workgroup: grid row y is sub-group y % per_group
    of group y // per_group, members m < n are sequences s0 + m.  Staged
    ids s_blk[m * ids + j] for j <= (ctx_m - 1) / B; the shared prefix
    covers the leading entries all usable members hold in common, capped at
    the shortest context; tiles of 16 tokens per segment (shared, then each
    member's own tokens) load token min(t, end - 1) from the segment's
    member's ids.  Every staged, loaded and written index is in bounds, every
    sequence is in exactly one workgroup, and each usable member's tokens
    0 .. ctx - 1 are each read exactly once, from the physical block its own
    table names.  With parts > 1 (grid z) each tile list is cut into `parts`
    contiguous ranges, one workgroup each, and every usable member's partial
    for each query head goes to workspace slot ((s * H + h) * parts + z)."""
    S, H, D = case.q.shape
    N, Hk, B, _ = case.k_cache.shape
    G = H // Hk
    sub = min(group, SIB_MAX // G)
    assert H % Hk == 0 and 2 <= group and sub >= 2  # matrix columns: members x query heads <= 16
    W = case.block_tables.shape[1]
    maxc = case.max_context_len
    assert maxc <= W * B
    ids = max(1, -(-maxc // B))
    assert sub * ids <= SIB_MAX_IDS
    cache_elems = N * Hk * B * D
    RPI = 64 * 8 // D
    per_group = -(-group // sub)
    rows = -(-S // group) * per_group
    covered = np.zeros(S, dtype=np.int64)
    for y in range(rows):
        gi, si = divmod(y, per_group)
        s0 = gi * group + si * sub
        n = min(sub, group - si * sub, S - s0)
        if n <= 0:
            continue
        covered[s0:s0 + n] += 1
        ctx = [int(case.context_lens[s0 + m]) for m in range(n)]
        usable = [0 < c <= maxc for c in ctx]
        blk = np.full((n, ids), -1, dtype=np.int64)
        for m in range(n):
            if usable[m]:
                nb = (ctx[m] - 1) // B + 1
                assert nb <= ids and nb <= W and (s0 + m) * W + nb - 1 < S * W
                row = case.block_tables[s0 + m, :nb].astype(np.int64)
                blk[m, :nb] = np.where((row >= 0) & (row < N), row, -1)
        members = [m for m in range(n) if usable[m]]
        if len(members) >= 2:
            minctx = min(ctx[m] for m in members)
            jmax = (minctx - 1) // B + 1
            common = jmax
            for j in range(jmax):
                if any(blk[m, j] != blk[members[0], j] for m in members):
                    common = j
                    break
            shared_end = min(common * B, minctx)
        else:
            shared_end = 0
        segs = [(0, shared_end, members[0] if members else 0, set(members))]
        segs += [(shared_end, ctx[m], m, {m}) for m in members]
        seen = {m: np.zeros(ctx[m], dtype=np.int64) for m in members}
        # the tile list, segment after segment, cut into `parts` ranges
        tiles = [(tb, tend, mid, cols) for tb0, tend, mid, cols in segs for tb in range(tb0, tend, SIB_TILE)]
        ntile = len(tiles)
        ranges = [(ntile * z // parts, ntile * (z + 1) // parts) for z in range(parts)]
        assert sum(hi - lo for lo, hi in ranges) == ntile and all(lo <= hi for lo, hi in ranges)
        for z in range(parts if parts > 1 else 0):
            for m in members:
                for hk in (0, Hk - 1):
                    slot = ((s0 + m) * H + hk * G + G - 1) * parts + z
                    assert slot < S * H * parts and (slot + 1) * D <= S * H * parts * D
        for tb, tend, mid, cols in (tiles[k] for lo, hi in ranges for k in range(lo, hi)):
            for i in range(SIB_TILE // RPI):
                t = np.minimum(tb + RPI * i + np.arange(RPI), tend - 1)
                assert (t >> int(np.log2(B))).max() < ids
                b = np.maximum(blk[mid, t // B], 0)
                e = b * Hk * B * D + (Hk - 1) * B * D + (t % B) * D + D - 8
                assert e.max() + 8 <= cache_elems
            # tokens this tile weighs (unmasked: tb + 4 g + j < tend)
            for t in range(tb, min(tb + SIB_TILE, tend)):
                for m in cols:
                    seen[m][t] += 1
                    # the block read is the member's own block for t
                    assert blk[mid, t // B] == blk[m, t // B]
        for m in members:
            assert (seen[m] == 1).all(), (y, m)
        # query operands and output rows: member c // G, query head hk G + c % G
        assert n * G <= SIB_MAX
        for col in range(n * G):
            row = (s0 + col // G) * H + (Hk - 1) * G + col % G
            assert row < S * H
        assert s0 + n - 1 < S
    assert (covered == 1).all()


@pytest.mark.parametrize("B", [8, 16, 32])
def test_siblings_parallel_sampling_bounds(B):
    case = wl.parallel_sampling(block_size=B)
    check_siblings_bounds(case, 4)


SIB_CASES = [
    # seed, group, dtype, D, B, prompts, samples, prompt_len, max_suffix
    (1, 2, "f16", 64, 1, 3, 2, 37, 20),
    (2, 3, "bf16", 128, 8, 4, 3, 100, 40),
    (3, 16, "f16", 128, 16, 2, 16, 70, 30),
    (4, 4, "bf16", 256, 32, 3, 4, 65, 64),
    (5, 5, "f16", 128, 256, 3, 4, 300, 10),  # groups cut across prompts
]


@pytest.mark.parametrize("seed,group,dtype,D,B,prompts,samples,plen,msuf", SIB_CASES)
def test_siblings_forked_bounds(seed, group, dtype, D, B, prompts, samples, plen, msuf):
    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=plen, num_heads=2,
                                head_dim=D, pool_tokens=max(4096, 64 * B), dtype=dtype, max_suffix=msuf)
    check_siblings_bounds(case, group)


@pytest.mark.parametrize("G,group,D", [(8, 4, 128), (8, 3, 128), (4, 8, 128), (2, 16, 128), (8, 16, 128),
                                       (4, 5, 128), (8, 4, 256), (4, 6, 64)])
def test_siblings_subgroup_bounds(G, group, D):
    """Groups cut into sub-groups of min(n, 16 // G) members."""
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=max(group, 4), prompt_len=90,
                                num_heads=2 * G, head_dim=D, pool_tokens=16384, max_suffix=40, num_kv_heads=2)
    check_siblings_bounds(case, group)


def test_siblings_wide_batch_bounds():
    """12000 unrelated short contexts in groups of 4 (G = 4: the 16 columns)."""
    case = dict(CASES)["wide-gqa"]()
    check_siblings_bounds(case, 4)


def test_siblings_unrelated_and_guarded_bounds():
    """Unrelated sequences (nothing shared), empty and impossible contexts,
    and an out-of-pool id in the shared region: still in bounds."""
    case = wl.random_case(77, 7, 2, 128, 16, "f16", ctx=[1, 300, 0, 17, 64, 65, 900], spare_blocks=4)
    check_siblings_bounds(case, 4)
    case.context_lens[2] = case.max_context_len + 5  # impossible: not staged
    check_siblings_bounds(case, 3)



@pytest.mark.parametrize("seed", range(16))
def test_random_siblings_case_bounds(seed):
    from test_gpu_random_cases import random_siblings_case

    case, group = random_siblings_case(seed)
    check_siblings_bounds(case, group)



@pytest.mark.parametrize("G,group", [(2, 4), (4, 4), (8, 2), (4, 3)])
def test_siblings_grouped_query_bounds(G, group):
    case = wl.parallel_sampling(block_size=16, num_prompts=3, samples=4, prompt_len=90, num_heads=2 * G, head_dim=128,
                                pool_tokens=8192, max_suffix=40, num_kv_heads=2)
    check_siblings_bounds(case, group)


def sibling_plan(S, H, Hk, D, B, group, maxc, ws_bytes, cus=256):
    """The host's choice for PA_DECODE_SIBLINGS(group): 0 = not taken,
    otherwise the number of workgroups each tile list is split over (1 =
    whole lists).  A thin grid (fewer workgroups than half the CUs) over
    contexts of 1024 tokens or more is split into about one workgroup per
    CU, at least 8 tiles of the longest context each, as many as the
    ungrouped plan's workspace holds (at least two); otherwise declined."""
    G = H // Hk
    sub = min(group, SIB_MAX // G)
    if group < 2 or sub < 2 or D < 64:
        return 0
    ids = max(1, -(-maxc // B))
    fits = sub * ids <= SIB_MAX_IDS
    rows = -(-S // group) * -(-group // sub)
    wgs = rows * Hk
    thin = 2 * wgs < cus and maxc >= 1024
    parts = 1
    if fits and thin:
        have = ws_bytes // (S * H * (D + 2) * 4)
        parts = min(-(-cus // wgs), have, -(-maxc // 128), 64)
    return (1 if not thin else parts) if fits and (not thin or parts >= 2) else 0


@pytest.mark.parametrize("Hk,samples,plen", [(8, 16, 1200), (32, 16, 1200), (8, 8, 4000), (2, 4, 2000)])
def test_siblings_split_bounds(Hk, samples, plen):
    """One prompt forked into samples, long enough for a thin grid: the tile
    lists are split over the workgroups the plain plan's workspace allows,
    every token of every member still read exactly once."""
    import paged_kv_cache_322_amd as pa

    H = 32 if Hk != 2 else 16
    case = wl.parallel_sampling(block_size=16, num_prompts=1, samples=samples, prompt_len=plen, num_heads=H,
                                head_dim=128, pool_tokens=32768, max_suffix=64, num_kv_heads=Hk)
    S, D = case.q.shape[0], case.q.shape[2]
    ws = pa.decode_workspace_size(S, H, D, case.max_context_len, num_kv_heads=Hk)
    parts = sibling_plan(S, H, Hk, D, 16, samples, case.max_context_len, ws)
    assert parts >= 2
    assert S * H * parts * (D + 2) * 4 <= ws
    check_siblings_bounds(case, samples, parts)


def test_sibling_plan_rule():
    """Not thin: whole lists; thin without a workspace: declined."""
    assert sibling_plan(256, 40, 40, 128, 16, 4, 756, 0) == 1  # config 4
    assert sibling_plan(16, 32, 8, 128, 16, 16, 4225, 0) == 0  # no room for partials
    assert sibling_plan(16, 32, 8, 128, 16, 16, 900, 0) == 1  # short contexts: whole lists
    assert sibling_plan(16, 32, 8, 128, 16, 16, 4225, 1 << 30) == 8  # 32 workgroups -> 1 per CU
    assert sibling_plan(16, 32, 8, 128, 16, 16, 4225, 3 * 16 * 32 * 130 * 4) == 3  # as the workspace holds
    assert sibling_plan(16, 32, 8, 128, 16, 16, 4225, 16 * 32 * 130 * 4) == 0  # room for one: declined


@pytest.mark.parametrize("dtype,D,B,H,Hk,prompts,samples,plen", [
    ("bf16", 256, 32, 4, 2, 1, 8, 1500), ("f16", 64, 8, 16, 4, 2, 8, 1100), ("bf16", 128, 16, 16, 2, 1, 4, 2100),
    ("f16", 128, 64, 4, 4, 3, 5, 1300)])
def test_siblings_split_shapes_bounds(dtype, D, B, H, Hk, prompts, samples, plen):
    """The split GPU cases at other head, block and group sizes."""
    import paged_kv_cache_322_amd as pa

    case = wl.parallel_sampling(block_size=B, num_prompts=prompts, samples=samples, prompt_len=plen, num_heads=H,
                                head_dim=D, pool_tokens=65536, max_suffix=48, num_kv_heads=Hk, dtype=dtype)
    S = case.q.shape[0]
    group = 4 if samples == 5 else samples
    ws = pa.decode_workspace_size(S, H, D, case.max_context_len, num_kv_heads=Hk)
    parts = sibling_plan(S, H, Hk, D, B, group, case.max_context_len, ws)
    assert parts >= 2, parts
    check_siblings_bounds(case, group, parts)


@pytest.mark.parametrize("seed", range(8))
def test_random_thin_siblings_bounds(seed):
    """The random thin-grid GPU cases, with the split count the host picks."""
    import paged_kv_cache_322_amd as pa
    from test_gpu_random_cases import random_thin_siblings_case

    case, group = random_thin_siblings_case(seed)
    S, H, D = case.q.shape
    Hk = case.k_cache.shape[1]
    ws = pa.decode_workspace_size(S, H, D, case.max_context_len, num_kv_heads=Hk)
    parts = sibling_plan(S, H, Hk, D, case.block_size, group, case.max_context_len, ws)
    if parts:
        check_siblings_bounds(case, group, parts)


def test_siblings_split_unrelated_bounds():
    """The thin split grid of unrelated sequences (empty and one-token
    contexts among them) that the GPU test runs."""
    import paged_kv_cache_322_amd as pa

    case = wl.random_case(91, 8, 4, 128, 16, "bf16", ctx=[1500, 1200, 0, 1100, 2000, 1, 1300, 1700], spare_blocks=4)
    ws = pa.decode_workspace_size(8, 4, 128, case.max_context_len)
    parts = sibling_plan(8, 4, 4, 128, 16, 8, case.max_context_len, ws)
    assert parts >= 2
    check_siblings_bounds(case, 8, parts)


def test_bench_sampling_one_bounds():
    """The benchmark's one-prompt workload (4000 tokens x 16 samples, 32 query
    over 8 K/V heads) under the split sibling grid the host picks, and under
    the ungrouped plan."""
    import paged_kv_cache_322_amd as pa

    case = wl.parallel_sampling(block_size=16, num_prompts=1, samples=16, prompt_len=4000, num_heads=32,
                                num_kv_heads=8, max_suffix=64)
    S, H, D = case.q.shape
    ws = pa.decode_workspace_size(S, H, D, case.max_context_len, num_kv_heads=8)
    parts = sibling_plan(S, H, 8, D, 16, 16, case.max_context_len, ws)
    assert parts == 8
    check_siblings_bounds(case, 16, parts)
    assert balanced_plan(S, 8, case.max_context_len, 4)  # the ungrouped plan (--siblings 0)
    for wgs in (512, 64):
        check_balanced_bounds(S, 8, 4, D, 16, case.k_cache.shape[0], case.block_tables.shape[1], case.context_lens,
                              case.block_tables, case.max_context_len, wgs)
