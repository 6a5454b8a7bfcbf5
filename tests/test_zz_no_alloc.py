"""pa_decode_static (the entry point that allocates nothing: split-K
partials in the library's static per-GPU scratch) through the C ABI, against
pa_decode with a caller workspace (same kernels: identical bits) and the
oracle (2e-3 for f16/bf16), on consecutive calls whose inputs shrink, and
its rejection of plans the scratch cannot hold."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_helpers import GpuCase, assert_close, log, oracle_decode, pa

pytestmark = pytest.mark.gpu


def static_vs_workspace(case, partition, strict=True):
    g = GpuCase(case)
    need = pa().decode_workspace_size(case.num_seqs, case.num_heads, case.head_dim, case.max_context_len,
                                      partition, case.num_kv_heads)
    log(f"{case.name}: partition={partition}, scratch needed {need} bytes")
    assert 0 < need <= pa().STATIC_SCRATCH_BYTES  # the split path, within the scratch
    ref_out = g.decode(partition=partition, out=torch.empty_like(g.q))
    out = torch.full_like(g.q, float("nan"))
    pa().decode_static(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len,
                       partition_size=partition)
    torch.cuda.synchronize()
    iv = torch.int32 if case.dtype == "f32" else torch.int16
    assert torch.equal(out.view(iv), ref_out.view(iv))
    assert_close(out, oracle_decode(case, case.k_cache, case.v_cache), case.dtype, f"{case.name} static",
                 strict=strict)


def test_static_scratch_two_calls_shrinking():
    # First a LLaMA-7B-shaped batch split into 256-token partitions (8.5 MB of
    # partials), then a small ragged batch with 64-token partitions: the
    # second call reuses the scratch the first one filled.
    static_vs_workspace(wl.llama7b_decode(), 256)
    static_vs_workspace(wl.random_case(901, 5, 4, 128, 16, "bf16", ctx=[1, 63, 64, 65, 700], spare_blocks=3), 64,
                        strict=False)


def test_static_scratch_balanced_split_then_smaller():
    # Grouped heads with few (sequence, K/V head) pairs: the balanced split
    # keeps its piece length in the scratch beside the partials.
    static_vs_workspace(wl.gqa_config("llama2-70b-tp8"), 0)
    static_vs_workspace(wl.random_case(902, 3, 8, 128, 16, "f16", ctx=[5, 300, 2000], num_kv_heads=1,
                                       spare_blocks=2), 0, strict=False)


def test_static_scratch_whole_contexts_need_none():
    case = wl.random_case(903, 4, 2, 64, 8, "f16", ctx=[1, 9, 100, 200], spare_blocks=2)
    g = GpuCase(case)
    out = torch.empty_like(g.q)
    pa().decode_static(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len)
    torch.cuda.synchronize()
    assert_close(out, oracle_decode(case, case.k_cache, case.v_cache), "f16", "static, no split", strict=False)


def test_static_scratch_rejects_plans_it_cannot_hold():
    # 512 sequences x 8 heads with 16-token partitions up to a 4096-token
    # bound need ~545 MB of partials: refused before any launch, out
    # untouched.  (The buffers are sized for the call, so it would be in
    # bounds even if it ran.)
    S, H, D, B, maxc = 512, 8, 128, 16, 4096
    rng = np.random.default_rng(904)
    case = wl.random_case(904, S, H, D, B, "f16", ctx=rng.integers(1, 20, S).tolist(), spare_blocks=2)
    g = GpuCase(case)
    width = maxc // B
    bt = torch.zeros((S, width), dtype=torch.int32, device="cuda")
    bt[:, : g.bt.shape[1]] = g.bt
    need = pa().decode_workspace_size(S, H, D, maxc, 16)
    assert need > pa().STATIC_SCRATCH_BYTES
    out = torch.full_like(g.q, 7.0)
    with pytest.raises(pa().PagedAttentionError) as ei:
        pa().decode_static(out, g.q, g.kc, g.vc, bt, g.ctx, case.scale, maxc, partition_size=16)
    torch.cuda.synchronize()
    assert ei.value.status == 6  # PA_ERR_SCRATCH
    assert (out.float() == 7.0).all()
