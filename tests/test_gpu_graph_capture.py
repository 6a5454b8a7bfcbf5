"""A decode step captured in a HIP graph: the newest tokens written by
pa_reshape_and_cache, then pa_decode_static (no workspace: split-K partials
in the library's static scratch) or pa_decode with a workspace allocated
before the capture.  The library enqueues kernels only (no allocation, no
memset), so the step can be captured.  The graph is replayed several times,
with eager work and synchronisation between the replays, and every replay
must reproduce the eager step bit for bit (the appended rows go to the same
slots with the same values each time).  Plans covered: whole contexts,
forced 256-token partitions (split + merge), the balanced split of a
grouped-query batch (pieces + merge), and a sibling-group decode split over
several workgroups (sibling kernel + merge)."""
import pytest
import torch

import workloads as wl
from gpu_helpers import GpuCase, log, pa

pytestmark = pytest.mark.gpu


def _case(plan):
    if plan == "balanced":
        return wl.gqa_config("llama2-70b-tp8", n_append=1)  # 128 (sequence, K/V head) pairs, G = 8
    return wl.llama7b_decode(n_append=1)


@pytest.mark.parametrize("entry", ["static", "workspace"])
@pytest.mark.parametrize("plan", ["whole", "split", "balanced"])
def test_graph_replay_of_a_decode_step(entry, plan):
    case = _case(plan)
    part = 256 if plan == "split" else 0
    g = GpuCase(case)
    assert len(g.steps) == 1 and g.steps[0][0] == "append"
    log(f"graph replay: {case.name}, entry {entry}, plan {plan}")
    ws = None
    if entry == "workspace":
        need = pa().decode_workspace_size(case.num_seqs, case.num_heads, case.head_dim, case.max_context_len, part,
                                          case.num_kv_heads)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(out):
        g.run_step(0)
        if entry == "static":
            pa().decode_static(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len,
                               partition_size=part)
        else:
            pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, partition_size=part,
                        workspace=ws)

    eager = torch.empty_like(g.q)
    step(eager)
    torch.cuda.synchronize()
    assert not torch.isnan(eager.float()).any()

    out = torch.full_like(g.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)  # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out)
    torch.cuda.synchronize()
    iv = torch.int16
    for r in range(4):
        out.fill_(float("nan"))
        junk = (eager.float() * 2.0).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(iv), eager.view(iv)), f"replay {r} differs from the eager step"
        del junk
    log(f"graph replay: 4 replays bitwise equal to the eager step")


@pytest.mark.parametrize("entry", ["static", "workspace"])
def test_graph_replay_of_split_sibling_decode(entry):
    """A sibling-group decode of one long prompt forked into 16 samples (a
    thin grid, split over several workgroups: the sibling kernel, then the
    merge kernel) captured and replayed, bit for bit as the eager call."""
    case = wl.parallel_sampling(block_size=16, num_prompts=1, samples=16, prompt_len=1200, num_heads=32,
                                head_dim=128, pool_tokens=32768, max_suffix=64, num_kv_heads=8)
    g = GpuCase(case)
    g.run_steps()
    S, H, D = case.q.shape
    ws = None
    if entry == "workspace":
        need = pa().decode_workspace_size(S, H, D, case.max_context_len, 0, 8)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    log(f"graph replay: {case.name}, siblings=16, entry {entry}")

    def step(out):
        if entry == "static":
            pa().decode_static(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, siblings=16)
        else:
            pa().decode(out, g.q, g.kc, g.vc, g.bt, g.ctx, case.scale, case.max_context_len, workspace=ws,
                        siblings=16)

    eager = torch.empty_like(g.q)
    step(eager)
    torch.cuda.synchronize()
    assert not torch.isnan(eager.float()).any()
    out = torch.full_like(g.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        junk = (eager.float() * 2.0).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs"
        del junk
