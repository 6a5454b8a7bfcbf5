#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = one serving decode step of a whole batch through the hot path:
``pa_reshape_and_cache`` stores every sequence's newest K/V row into its
slot, then ``pa_decode`` attends each sequence's query over its paged
context (partition kernel, plus the merge kernel for contexts longer than a
partition).  The default workload is the LLaMA-7B-shaped decode layer: 64
sequences, context lengths uniform in [128, 2048], 32 heads, head_dim 128,
fp16, 16-token blocks in an 8192-block pool with random physical placement.
The workload has no shared blocks, so copy-on-write has nothing to copy in
the step; ``pa_copy_blocks`` is timed beside it on a batch of block pairs.

Reported (one JSON line on stdout):
  value       algorithmic bytes of the step / step time (GB/s), with
              bytes = 2*e*H*D*sum(ctx) (K and V) + 2*S*H*D*e (q, out)
                      + 4*sum(ceil(ctx/B)) (block ids) + 4*S (lengths)
                      + 4*T*H*D*e + 8*T (append: read k/v, write k/v, slots)
  roofline    pa_decode alone: its algorithmic bytes / its average duration
              over a loop of launches (HIP events around the loop, on the
              launch stream), against the 8 TB/s HBM3E peak
  cpu_baseline the float64 CPU oracle on the same batch, on this host

Inputs are resident in HBM before timing.  Consecutive steps alternate
between ``--rotate`` independent copies of the KV pools so no step finds the
previous step's blocks in the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "paged decode attention: KV-read GB/s and % of HBM peak; decode tokens/s"
SWAP_WORKLOAD = ("swap-llama7b: preempt 16 of the 64 LLaMA-7B-shaped decode sequences: swap their "
                 "K/V blocks out to a pinned host pool and back in under new ids; H=32, D=128, f16, B=16")
LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction, nominal
WORKLOADS = {
    "llama7b": "llama7b-decode-layer: 64 seqs, ctx U[128,2048], H=32, D=128, f16, B=16, 8192-block pool",
    "opt13b": "opt13b-decode-layer: 256 seqs, ctx lognormal(median 300, sigma 0.9) in [16,2048], H=40, D=128, f16, B=16",
    "sampling": "parallel-sampling-cow: 64 prompts x 4 samples, prompt 500, suffix U[0,256], H=40, D=128, f16",
    "sampling-gqa": "parallel-sampling-cow-gqa: 64 prompts x 4 samples, prompt 500, suffix U[0,256], 32 query / 8 K/V "
                    "heads (LLaMA-3-8B-shaped), D=128, f16",
    "sampling-70b": "parallel-sampling-cow-70b: 64 prompts x 4 samples, prompt 500, suffix U[0,256], 64 query / 8 K/V "
                    "heads (LLaMA-2-70B-shaped), D=128, f16",
    "sampling-one": "parallel-sampling-one-prompt: 1 prompt x 16 samples, prompt 4000, suffix U[0,64], 32 query / 8 K/V "
                    "heads (LLaMA-3-8B-shaped), D=128, f16",
    "opt175b": "opt175b-decode-layer: 128 seqs, ctx U[1024,2048], H=96, D=128, bf16, B=16, 16384-block pool",
    "opt175b-tp8": "opt175b-decode-tp8-share: the OPT-175B-shaped layer with the 12 of its 96 heads one of 8 tensor-parallel GPUs holds; "
            "128 seqs, ctx U[1024,2048], D=128, bf16, B=16, 16384-block pool",
    "gqa8b": "llama3-8b-gqa-decode-layer: 64 seqs, ctx U[128,2048], 32 query / 8 K/V heads, D=128, f16, B=16",
    "gqa70b": "llama2-70b-gqa-tp8-share: 128 seqs, ctx U[512,4096], 8 query / 1 K/V head, D=128, bf16, B=16",
    "prefill-llama7b": "llama7b-chunked-prefill: 16 seqs x 512-token chunks over cached prefixes U[0,1536], H=32, "
                       "D=128, f16, B=16",
    "prefill-gqa8b": "llama3-8b-chunked-prefill: 16 seqs x 512-token chunks over cached prefixes U[0,1536], "
                     "32 query / 8 K/V heads, D=128, f16, B=16",
    "prefill-prompts": "llama7b-prompt-prefill: 32 whole prompts, lognormal(median 300, sigma 0.9) lengths in "
                       "[16,2048], H=32, D=128, bf16, B=16",
    "swap": SWAP_WORKLOAD,
    "block-manager": "block-manager: host bookkeeping of a decode step for the OPT-13B-shaped batch's 256 sequences "
                     "(lognormal(300, 0.9) contexts, B=16) and prefix-cached admission of 256 prompts sharing a "
                     "512-token system prompt",
}
SAMPLING_KINDS = ("sampling", "sampling-gqa", "sampling-70b", "sampling-one")  # forked samples sharing prompt blocks
PREFILL_KINDS = {"prefill-llama7b": "llama7b", "prefill-gqa8b": "llama3-8b", "prefill-prompts": "prompts"}
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, vendor figure
PREFILL_METRIC = "paged prefill attention: TFLOP/s and % of MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed warmup steps (default 100: after an idle period, such as the workload set-up, "
                         "sustained load runs slow for the first ~10-15 ms while the clocks ramp; measured on the "
                         "parallel-sampling decode step, 289 us after 10 warmup steps, 260 us after 100)")
    ap.add_argument("--config", default="llama7b", choices=sorted(WORKLOADS))
    ap.add_argument("--partition", type=int, default=0, help="KV partition tokens (0 = library default)")
    ap.add_argument("--block-size", type=int, default=16, help="block size of the parallel-sampling workload (8, 16 or 32)")
    ap.add_argument("--shared-blocks", choices=["auto", "on", "off"], default="auto",
                    help="PA_DECODE_SHARED_BLOCKS (cached K/V loads); auto = on for the parallel-sampling workload "
                         "decoded without sibling groups (its samples then re-read the shared prompt blocks)")
    ap.add_argument("--siblings", default="auto",
                    help="PA_DECODE_SIBLINGS group size (0 = off); auto = the samples per prompt (4, or 16 for "
                         "sampling-one) for the parallel-sampling workloads, off otherwise")
    ap.add_argument("--rotate", type=int, default=2, help="independent pool copies cycled across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second-config", action="store_true",
                    help="with the default workload, skip timing the OPT-13B-shaped batch beside it")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle baseline")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_case(cfg, block_size=16):
    import workloads as wl

    if cfg == "llama7b":
        return wl.llama7b_decode(n_append=1)
    if cfg == "opt13b":
        return wl.opt13b_decode()
    if cfg == "sampling":
        return wl.parallel_sampling(block_size=block_size)
    if cfg == "sampling-gqa":
        return wl.parallel_sampling(block_size=block_size, num_heads=32, num_kv_heads=8)
    if cfg == "sampling-70b":
        return wl.parallel_sampling(block_size=block_size, num_heads=64, num_kv_heads=8)
    if cfg == "sampling-one":
        return wl.parallel_sampling(block_size=block_size, num_prompts=1, samples=16, prompt_len=4000, num_heads=32,
                                    num_kv_heads=8, max_suffix=64)
    if cfg == "gqa8b":
        return wl.gqa_config("llama3-8b", n_append=1)
    if cfg == "gqa70b":
        return wl.gqa_config("llama2-70b-tp8", n_append=1)
    if cfg in PREFILL_KINDS:
        return wl.prefill_config(PREFILL_KINDS[cfg])
    if cfg == "swap":
        return wl.llama7b_decode()
    if cfg == "block-manager":
        return None
    if cfg == "opt175b-tp8":
        return wl.opt175b_decode(num_heads=12, n_append=1)
    return wl.opt175b_decode(n_append=1)


def algorithmic_bytes(case, timed_steps):
    """(decode bytes, store bytes) of one step.

    decode: K and V of every context token (the newest token's included,
    wherever it is read from), q, out, block ids, context lengths.
    store: writing the newest tokens' K and V rows into the caches.
    """
    e = case.elem_bytes
    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    Hk = case.num_kv_heads  # K/V heads (H / G with grouped-query attention)
    ctx = case.context_lens.astype(np.int64)
    decode = 2 * e * Hk * D * int(ctx.sum()) + 2 * S * H * D * e + 4 * int(np.ceil(ctx / B).sum()) + 4 * S
    T = sum(st.slot_mapping.size for st in timed_steps)
    store = 2 * T * Hk * D * e
    return decode, store


def unique_kv_bytes(case):
    """K+V bytes of the distinct (block, slot) positions the decode reads:
    blocks shared by several sequences count once."""
    B = case.block_size
    seen = {}
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        for j in range(-(-n // B)):
            b = int(case.block_tables[s, j])
            seen[b] = max(seen.get(b, 0), min(B, n - j * B))
    return 2 * case.elem_bytes * case.num_kv_heads * case.head_dim * sum(seen.values())


# Committed HBM counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled
# by a copy kernel of known size), per workload at its default plan.
COUNTER_FILES = {"llama7b": "decode_llama7b_counters.txt", "opt13b": "decode_opt13b_counters.txt",
                 "sampling": "decode_parallel_sampling_b16_counters.txt",
                 "sampling-gqa": "decode_parallel_sampling_gqa_counters.txt",
                 "sampling-70b": "decode_parallel_sampling_70b_counters.txt", "opt175b": "decode_opt175b_counters.txt",
                 "gqa8b": "decode_gqa_llama3_8b_counters.txt", "gqa70b": "decode_gqa_llama2_70b_tp8_counters.txt",
                 "prefill-llama7b": "prefill_llama7b_counters.txt", "prefill-gqa8b": "prefill_gqa_llama3_8b_counters.txt",
                 "prefill-prompts": "prefill_prompts_bf16_counters.txt"}
DECODE_SOURCES = ("pa_decode_impl.h", "pa_decode_mfma.h", "pa_decode_siblings.h", "pa_device.h", "pa_internal.h")
PREFILL_SOURCES = ("pa_prefill.hip", "pa_decode_mfma.h", "pa_device.h", "pa_internal.h")


def traffic_from_profiles(config, kernel_src_sha):
    """HBM bytes per decode launch from the committed counter summary of this
    workload, if it was taken on the current kernel source; else None."""
    if config not in COUNTER_FILES:
        return None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", COUNTER_FILES[config])
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_src_sha:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_kernel_name(case, siblings=0):
    """The decode kernel the library runs for this shape: the sibling-group
    kernel when siblings are named and it is built for the shape, the
    matrix-core kernel for 16-bit caches with D in {64, 128, 256} and grouped
    heads, else the vector-ALU kernel."""
    G = case.num_heads // case.num_kv_heads
    mfma_shape = case.elem_bytes == 2 and case.head_dim in (64, 128, 256)
    if mfma_shape and siblings >= 2 and min(siblings, 16 // G) >= 2:
        return "decode_siblings_kernel"
    if mfma_shape and G >= 2:
        return "decode_mfma_kernel"
    return "decode_partition_kernel"


def kernel_source_sha(sources=DECODE_SOURCES):
    import hashlib

    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_322_amd", "csrc")
    h = hashlib.sha256()
    for name in sources:
        h.update(open(os.path.join(root, name), "rb").read())
    return h.hexdigest()


def cpu_baseline(case, target_s, timed_steps, setup_pools=None):
    """The float64 oracle on the same kind of step, on a bounded sample.

    Times oracle.reshape_and_cache (the sample's new rows; the oracle copies
    the whole pool each call, as it stands) followed by oracle.paged_decode,
    for the first k sequences of the batch, with k the whole batch when that
    fits about a third of ``target_s`` and fewer otherwise.  Repeats until
    ``target_s`` of CPU time or 10 runs and reports the best run, as GB/s over
    the same algorithmic bytes the GPU figure uses (restricted to the sample).
    """
    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    k0, v0 = setup_pools if setup_pools is not None else (case.k_cache, case.v_cache)
    for st in timed_steps:
        assert st.slot_mapping.size == case.num_seqs  # one new row per sequence, in sequence order

    def run(k):
        t0 = time.perf_counter()
        kc, vc = k0, v0
        for st in timed_steps:
            kc, vc = oracle.reshape_and_cache(st.key[:k], st.value[:k], kc, vc, st.slot_mapping[:k])
        oracle.paged_decode(case.q[:k], kc, vc, case.block_tables[:k], case.context_lens[:k], case.scale,
                            case.dtype)
        return time.perf_counter() - t0

    S = case.num_seqs
    # The oracle's append copies the whole pool (a fixed cost); the decode
    # cost grows with the sequences sampled.  Size k from both.
    t0 = time.perf_counter()
    for st in timed_steps:
        oracle.reshape_and_cache(st.key[:1], st.value[:1], k0, v0, st.slot_mapping[:1])
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.paged_decode(case.q[:1], k0, v0, case.block_tables[:1], case.context_lens[:1], case.scale, case.dtype)
    t_seq = max(time.perf_counter() - t0, 1e-4) * float(case.context_lens.mean()) / max(1, int(case.context_lens[0]))
    budget = target_s / 3 - t_fixed
    k = S if t_fixed + t_seq * S <= target_s / 3 else max(1, min(S, int(budget / t_seq)))
    best, total, reps = math.inf, 0.0, 0
    while reps < 10 and (reps < 2 or total < target_s):
        dt = run(k)
        best, total, reps = min(best, dt), total + dt, reps + 1
    e = case.elem_bytes
    H, Hk, D, B = case.num_heads, case.num_kv_heads, case.head_dim, case.block_size
    ctx = case.context_lens[:k].astype(np.int64)
    nbytes = 2 * e * Hk * D * int(ctx.sum()) + 2 * k * H * D * e + 4 * int(np.ceil(ctx / B).sum()) + 4 * k
    nbytes += sum(2 * k * Hk * D * e for _ in timed_steps)
    return {
        "value": round(nbytes / best / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"first {k} of {S} sequences ({'append + ' if timed_steps else ''}decode), best of {reps} runs "
                  f"({best:.2f} s each; float64 numpy, BLAS threads {blas_threads}; host has "
                  f"{len(os.sched_getaffinity(0))} cpus)",
        "seconds_per_run": round(best, 4),
        "sample_bytes": int(nbytes),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the paged "
              "decode path has no cross-GPU step; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_kv_cache_322_amd as pa

    dev = torch.device("cuda:0")
    if args.config == "block-manager":
        return bench_block_manager(args)
    log(f"building workload config {args.config}")
    case = make_case(args.config, args.block_size)
    if args.config in PREFILL_KINDS:
        return bench_prefill(args, case, pa, torch, dev)
    if args.config == "swap":
        return bench_swap(args, case, pa, torch, dev)
    result = bench_decode(args, args.config, case, pa, torch, dev, full=True)
    del case
    if args.config == "llama7b" and not args.no_second_config:
        # The OPT-13B-shaped batch (chat-like lengths, one appended token
        # per sequence) timed the same way in the same run, with its own
        # pools (freed after).
        log("building workload config opt13b")
        second = bench_decode(args, "opt13b", make_case("opt13b"), pa, torch, dev, full=False)
        result["configs"] = {"opt13b": second}
    probe = hbm_read_probe(pa, torch, dev)
    result["hbm_read_probe"] = probe
    best = probe["best_GB/s"]
    result["roofline"]["frac_of_read_probe"] = round(result["roofline"]["achieved"] / best, 4)
    result["roofline"]["frac_of_scattered_read_probe"] = round(
        result["roofline"]["achieved"] / probe["scattered_best_GB/s"], 4)
    for extra in result.get("configs", {}).values():
        extra["roofline_frac_of_read_probe"] = round(extra["roofline_achieved"] / best, 4)
        extra["roofline_frac_of_scattered_read_probe"] = round(
            extra["roofline_achieved"] / probe["scattered_best_GB/s"], 4)
    print(json.dumps(result), flush=True)


def hbm_read_probe(pa, torch, dev, gib=4, reps=10):
    """Achievable streaming-read rate (``pa_hbm_read_probe``): one 4 GiB
    buffer read once per launch with 16-byte loads, over a few shapes
    (non-temporal or cached loads, grid size, grid-stride or contiguous runs
    per workgroup); the best is the measured read ceiling decode is quoted
    against beside the vendor peak."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(cus * 8, dtype=torch.int32, device=dev)
    runs = []
    # (non-temporal, workgroups per CU, contiguous run bytes (0 = grid-stride), runs in a scattered order)
    shapes = [(True, 8, 0, False), (False, 8, 0, False), (True, 2, 65536, False), (True, 4, 65536, False),
              (True, 8, 65536, False), (True, 4, 8192, False), (True, 8, 8192, False), (True, 4, 262144, False),
              (False, 4, 65536, False), (True, 4, 8192, True), (True, 8, 8192, True), (True, 4, 16384, True)]
    for nt, per_cu, run, sc in shapes:
        wgs = cus * per_cu
        for _ in range(3):
            pa.hbm_read_probe(buf, sink, wgs, nontemporal=nt, run_bytes=run, scattered=sc)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            pa.hbm_read_probe(buf, sink, wgs, nontemporal=nt, run_bytes=run, scattered=sc)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        runs.append({"nontemporal": nt, "workgroups": wgs, "run_bytes": run, "scattered": sc, "us": round(us, 1),
                     "GB/s": round(buf.numel() / us / 1e3, 1)})
    del buf
    best = max(runs, key=lambda r: r["GB/s"])
    best_sc = max((r for r in runs if r["scattered"]), key=lambda r: r["GB/s"])
    log(f"HBM read probe: best {best}; scattered 8-16 KB runs {best_sc}")
    return {"bytes": gib << 30, "best_GB/s": best["GB/s"], "best": best,
            "scattered_best_GB/s": best_sc["GB/s"], "scattered_best": best_sc, "runs": runs,
            "note": "pa_hbm_read_probe: every byte of a 4 GiB buffer read once per launch (512-thread "
                    "workgroups, 16-byte loads, four in flight per lane; grid-stride or contiguous runs per "
                    "workgroup, in order or scattered as paged blocks are); HIP events around 10 launches; the best "
                    "shape is the ceiling, and the best scattered 8-16 KB-run shape the ceiling for decode's "
                    "access pattern"}


def bench_decode(args, config, case, pa, torch, dev, full=True):
    """The decode step of one workload.  full: the complete JSON record (copy
    probe, CPU baseline); otherwise a summary for the record's `configs`."""
    import workloads as wl

    # The parallel-sampling workload's prompt write, fork copies and suffix
    # writes are set-up; the other workloads time their one-token-per-sequence
    # append with the decode.
    if config in SAMPLING_KINDS:
        setup_steps, timed_steps = list(case.steps), []
    else:
        setup_steps, timed_steps = [], list(case.steps)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]

    def up(a):
        a = np.ascontiguousarray(a)
        if case.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    q, bt, ctx = up(case.q), up(case.block_tables), up(case.context_lens)
    appends = [(up(st.key), up(st.value), up(st.slot_mapping)) for st in timed_steps]
    pools = []
    for _ in range(max(1, args.rotate)):
        kc, vc = up(case.k_cache), up(case.v_cache)
        for st in setup_steps:
            if isinstance(st, wl.AppendStep):
                pa.reshape_and_cache(up(st.key), up(st.value), kc, vc, up(st.slot_mapping))
            else:
                pa.copy_blocks(kc, vc, up(st.pairs))
        pools.append((kc, vc))
    out = torch.empty_like(q)
    max_ctx = case.max_context_len
    ws_bytes = pa.decode_workspace_size(S, H, D, max_ctx, args.partition, case.num_kv_heads)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    siblings = (int(case.meta["samples"]) if config in SAMPLING_KINDS else 0) if args.siblings == "auto" \
        else int(args.siblings)
    # Cached K/V loads pay off when several workgroups read the same blocks:
    # the parallel-sampling workload decoded without sibling groups.  With
    # them, each shared block is read once per (group, head) and the
    # non-temporal loads are faster (measured: 229 -> 206 us at B = 16).
    shared = args.shared_blocks == "on" or (args.shared_blocks == "auto" and config in SAMPLING_KINDS and siblings < 2)
    fused = bool(timed_steps)
    if fused:
        assert len(timed_steps) == 1 and timed_steps[0].slot_mapping.size == S  # one newest row per sequence
        k_new, v_new, slots = appends[0]

    def step_fused(i, ev=None):
        kc, vc = pools[i % len(pools)]
        if ev is not None:
            ev[0].record()
        pa.append_decode(out, q, k_new, v_new, kc, vc, bt, ctx, case.scale, max_ctx,
                         partition_size=args.partition, workspace=ws, shared_blocks=shared)
        if ev is not None:
            ev[1].record()

    def step_two(i, ev=None):
        kc, vc = pools[i % len(pools)]
        if ev is not None:
            ev[0].record()
        for kn, vn, sl in appends:
            pa.reshape_and_cache(kn, vn, kc, vc, sl)
        if ev is not None:
            ev[1].record()
        pa.decode(out, q, kc, vc, bt, ctx, case.scale, max_ctx, partition_size=args.partition, workspace=ws,
                  shared_blocks=shared, siblings=siblings)
        if ev is not None:
            ev[2].record()

    medians = []  # per run: median over the steps of each event-pair span

    def run(step, nev):
        """Step time from an uninstrumented pass; per-launch times from a
        second pass with HIP events around each launch."""
        for i in range(args.warmup):
            step(i)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            step(i)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        spans = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(nev - 1)]
        medians.append([float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(nev - 1)])
        return ms, spans

    log(f"warmup {args.warmup} steps, then {args.steps} timed steps")
    ms_step, (append_ms, launch_ms) = run(step_two, 3)
    log(f"step {ms_step*1e3:.1f} us (append {append_ms*1e3:.1f} us, decode {launch_ms*1e3:.1f} us)")
    if fused:
        fused_ms, (fused_launch_ms,) = run(step_fused, 2)
        log(f"fused step {fused_ms*1e3:.1f} us (launch {fused_launch_ms*1e3:.1f} us)")

    # pa_decode alone, timed over a loop without per-launch events: on the
    # rotated pool copies, and back-to-back on one copy (a launch may then find
    # blocks the previous one left in the last-level cache or the TLBs).
    # Reported beside the value; never used as it.
    def decode_loop(reps, rotate):
        def one(i):
            kc, vc = pools[i % len(pools)] if rotate else pools[0]
            pa.decode(out, q, kc, vc, bt, ctx, case.scale, max_ctx, partition_size=args.partition, workspace=ws,
                      shared_blocks=shared, siblings=siblings)
        for i in range(3):
            one(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            one(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    rot_ms = decode_loop(args.steps, True)
    b2b_ms = decode_loop(args.steps, False)
    log(f"decode loop: rotated {rot_ms*1e3:.1f} us, back-to-back {b2b_ms*1e3:.1f} us")

    decode_bytes, store_bytes = algorithmic_bytes(case, timed_steps)
    step_bytes = decode_bytes + store_bytes
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # The dominant kernel's average duration: a loop of pa_decode launches on
    # the rotated pool copies, bracketed by HIP events on the launch stream
    # (per-launch event pairs add their own ~2-4 us to each launch).
    achieved = decode_bytes / (rot_ms * 1e-3) / 1e9
    if not full:
        return {
            "workload": WORKLOADS[config],
            "step": "pa_reshape_and_cache (1 new token per sequence) + pa_decode" if fused else "pa_decode",
            "GB/s": round(value, 1),
            "ms_per_step": round(ms_step, 5),
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
            "decode_tokens_per_s": round(S / (ms_step * 1e-3), 1),
            "step_bytes": int(step_bytes),
            "roofline_achieved": round(achieved, 1),
            "roofline_frac": round(achieved / HBM_PEAK_GBPS, 4),
            "avg_launch_us": round(rot_ms * 1e3, 2),
            "back_to_back_us": round(b2b_ms * 1e3, 2),
            "fused_ms_per_step": round(fused_ms, 5) if fused else None,
            "fused_GB/s": round(step_bytes / (fused_ms * 1e-3) / 1e9, 1) if fused else None,
            "dtype": case.dtype,
            "num_seqs": S,
            "sum_context_len": int(case.context_lens.sum()),
            "partition_tokens": pa.partition_tokens(S, H, max_ctx, args.partition, num_kv_heads=case.num_kv_heads),
        }

    # Copy-on-write block copies, timed beside the step on the first pool:
    # a fork-sized batch (192 pairs) and a large batch used as the HBM copy probe.
    used = np.unique(case.block_tables[case.block_tables >= 0])
    free = np.setdiff1d(np.arange(case.num_blocks), used)
    block_bytes = case.num_kv_heads * B * D * case.elem_bytes

    def time_copies(n, reps=20):
        n = int(min(n, used.size, free.size))
        pairs = up(np.stack([used[:n], free[:n]], axis=1).astype(np.int64))
        kc, vc = pools[0]
        pa.copy_blocks(kc, vc, pairs)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            pa.copy_blocks(kc, vc, pairs)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        moved = 2 * 2 * n * block_bytes  # K and V, read and write
        return {"pairs": n, "us": round(us, 2), "GB/s": round(moved / us / 1e3, 1)}

    cow = time_copies(192)
    probe = time_copies(4096)
    log(f"copy_blocks: {cow}; copy probe: {probe}")

    # The committed counters cover each profiled workload at its default partition.
    default_part = pa.partition_tokens(S, H, max_ctx, num_kv_heads=case.num_kv_heads)
    # The parallel-sampling counters were taken at its default 16-token blocks.
    profiled = args.partition in (0, default_part) and (config != "sampling" or B == 16)
    traffic = traffic_from_profiles(config, kernel_source_sha()) if profiled else None

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[config],
            "step": ("pa_reshape_and_cache (1 new token per sequence) + pa_decode" if fused else
                     "pa_decode (prompt write, copy-on-write fork and suffix writes done before timing)"),
            "num_seqs": S,
            "num_heads": H,
            "num_kv_heads": case.num_kv_heads,
            "head_dim": D,
            "block_size": B,
            "num_blocks": case.num_blocks,
            "sum_context_len": int(case.context_lens.sum()),
            "max_context_len": max_ctx,
            "partition_tokens": pa.partition_tokens(S, H, max_ctx, args.partition, num_kv_heads=case.num_kv_heads),
            "pool_copies_rotated": len(pools),
            "shared_blocks_flag": shared,
            "siblings_flag": siblings,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "step_bytes": int(step_bytes),
        "roofline": {
            "kernel": f"pa_decode ({decode_kernel_name(case, siblings)}, plus decode_merge_kernel when a context is "
                      "split): HIP events around a loop of launches on the rotated pool copies",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(decode_bytes),
            "avg_launch_us": round(rot_ms * 1e3, 2),
            "event_pair_per_launch_us": round(launch_ms * 1e3, 2),
            "event_pair_median_us": round(medians[0][1] * 1e3, 2),
        },
        "append_us": round(append_ms * 1e3, 2) if fused else None,
        "fused": ({"entry_point": "pa_append_decode", "ms_per_step": round(fused_ms, 5),
                   "GB/s": round(step_bytes / (fused_ms * 1e-3) / 1e9, 1),
                   "launch_us": round(fused_launch_ms * 1e3, 2)} if fused else None),
        "decode_loop": {"rotated_us": round(rot_ms * 1e3, 2),
                        "rotated_GB/s": round(decode_bytes / (rot_ms * 1e-3) / 1e9, 1),
                        "back_to_back_us": round(b2b_ms * 1e3, 2),
                        "back_to_back_GB/s": round(decode_bytes / (b2b_ms * 1e-3) / 1e9, 1),
                        "note": "pa_decode alone in a loop without per-launch events, on the rotated pool copies "
                                "and repeated on one copy; not the value"},
        "copy_blocks": cow,
        "hbm_copy_probe": probe,
    }
    if config in SAMPLING_KINDS:
        ub = unique_kv_bytes(case)
        result["unique_kv_bytes"] = int(ub)
        result["unique_kv_GBps"] = round(ub / (rot_ms * 1e-3) / 1e9, 1)
        result["kv_memory_saved_by_sharing"] = round(case.meta["kv_memory_saved"], 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same batch")
        setup_pools = None
        if setup_steps:
            import oracle

            kc, vc = case.k_cache, case.v_cache
            for st in setup_steps:
                if isinstance(st, wl.AppendStep):
                    kc, vc = oracle.reshape_and_cache(st.key, st.value, kc, vc, st.slot_mapping)
                else:
                    kc, vc = oracle.copy_blocks(kc, vc, st.pairs)
            setup_pools = (kc, vc)
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, timed_steps, setup_pools)
        result["cpu_baseline"]["gpu_over_oracle"] = round(value / result["cpu_baseline"]["value"], 1)
    return result


def prefill_flops(case, seqs=None):
    """Algorithmic flops of one prefill call: for every query row at position
    p and every head, 2*D for q.k and 2*D for p.v over the p + 1 keys it
    attends to."""
    n = case.query_lens
    ctx = case.context_lens.astype(np.int64)
    idx = range(case.num_seqs) if seqs is None else seqs
    pairs = 0
    for s in idx:
        first = int(ctx[s] - n[s])
        pairs += int(n[s]) * (first + 1) + int(n[s]) * (int(n[s]) - 1) // 2
    return 4 * case.head_dim * case.num_heads * pairs


def cpu_baseline_prefill(case, target_s):
    """The float64 oracle on the host for the first k sequences of the batch:
    oracle.reshape_and_cache of their chunk rows, then oracle.paged_prefill,
    with k sized so one run takes about a third of ``target_s``.  Reported as
    TFLOP/s over the same algorithmic flops the GPU figure uses."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    st = case.steps[0]
    qs = case.query_start

    def run(k):
        t0 = time.perf_counter()
        r1 = int(qs[k])
        kc, vc = oracle.reshape_and_cache(st.key[:r1], st.value[:r1], case.k_cache, case.v_cache,
                                          st.slot_mapping[:r1])
        oracle.paged_prefill(case.q[:r1], kc, vc, case.block_tables[:k], case.context_lens[:k], qs[: k + 1],
                             case.scale, case.dtype)
        return time.perf_counter() - t0

    t1 = run(1)
    per_flop = t1 / max(1, prefill_flops(case, [0]))
    k = 1
    while k < case.num_seqs and per_flop * prefill_flops(case, range(k + 1)) <= target_s / 3:
        k += 1
    best, total, reps = math.inf, 0.0, 0
    while reps < 5 and (reps < 2 or total < target_s):
        dt = run(k)
        best, total, reps = min(best, dt), total + dt, reps + 1
    flops = prefill_flops(case, range(k))
    return {
        "value": round(flops / best / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"first {k} of {case.num_seqs} sequences (chunk append + prefill), best of {reps} runs "
                  f"({best:.2f} s each; float64 numpy, BLAS threads {blas_threads}; host has "
                  f"{len(os.sched_getaffinity(0))} cpus)",
        "seconds_per_run": round(best, 4),
        "sample_flops": int(flops),
    }


def bench_prefill(args, case, pa, torch, dev):
    """One step = pa_reshape_and_cache of every sequence's chunk K/V, then
    pa_prefill of the chunk queries over the paged context."""

    def up(a):
        a = np.ascontiguousarray(a)
        if case.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    st = case.steps[0]
    q, bt, ctx, qs = up(case.q), up(case.block_tables), up(case.context_lens), up(case.query_start)
    kn, vn, slots = up(st.key), up(st.value), up(st.slot_mapping)
    pools = [(up(case.k_cache), up(case.v_cache)) for _ in range(max(1, args.rotate))]
    out = torch.empty_like(q)
    mq, mc = int(case.query_lens.max()), case.max_context_len
    torch.cuda.synchronize()

    def step(i, ev=None):
        kc, vc = pools[i % len(pools)]
        if ev is not None:
            ev[0].record()
        pa.reshape_and_cache(kn, vn, kc, vc, slots)
        if ev is not None:
            ev[1].record()
        pa.prefill(out, q, kc, vc, bt, ctx, qs, case.scale, mq, mc)
        if ev is not None:
            ev[2].record()

    log(f"warmup {args.warmup} steps, then {args.steps} timed steps")
    for i in range(args.warmup):
        step(i)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    append_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    launch_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    log(f"step {ms_step*1e3:.1f} us (append {append_ms*1e3:.1f} us, prefill {launch_ms*1e3:.1f} us)")

    flops = prefill_flops(case)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    traffic = traffic_from_profiles(args.config, kernel_source_sha(PREFILL_SOURCES))
    e = case.elem_bytes
    Hk = case.num_kv_heads
    kv_bytes = 2 * e * Hk * D * int(case.context_lens.astype(np.int64).sum())
    result = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.config],
            "step": "pa_reshape_and_cache (the chunks' K/V rows) + pa_prefill",
            "num_seqs": S,
            "num_heads": H,
            "num_kv_heads": Hk,
            "head_dim": D,
            "block_size": B,
            "num_blocks": case.num_blocks,
            "query_rows": case.num_tokens,
            "sum_context_len": int(case.context_lens.sum()),
            "max_query_len": mq,
            "max_context_len": mc,
        },
        "pct_of_mfma_peak": round(100 * value / MFMA_PEAK_TFLOPS, 2),
        "prefill_tokens_per_s": round(case.num_tokens / (ms_step * 1e-3), 1),
        "step_flops": int(flops),
        "roofline": {
            "kernel": "pa_prefill (prefill_kernel), event-timed",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": int(flops),
            "avg_launch_us": round(launch_ms * 1e3, 2),
            "kv_bytes_read_once": int(kv_bytes),
        },
        "append_us": round(append_ms * 1e3, 2),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the batch")
        result["cpu_baseline"] = cpu_baseline_prefill(case, args.cpu_seconds)
        result["cpu_baseline"]["gpu_over_oracle"] = round(value / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)


def bench_block_manager(args):
    """Host-side cost of the library's C++ block manager, against the Python
    reference model doing the same operations.

    Decode step: the OPT-13B-shaped batch's 256 sequences (contexts lognormal(300, 0.9) in
    [16, 2048], B = 16) each take one token (pa_bm_append_batch: slots and
    copy pairs), then the step's block tables are exported
    (pa_bm_block_tables).  Admission: 256 prompts of a 512-token shared system
    prompt plus 64 own tokens enter with prefix caching (32 whole blocks
    reused each) and reserve their own tokens."""
    from paged_kv_cache_322_amd.block_manager import BlockManager
    from oracle.block_manager import BlockManagerModel
    import workloads as wl

    lens = wl.opt13b_context_lengths()
    S, B = len(lens), 16
    steps = max(20, args.steps)
    grow = -(-(steps + B) // B)  # blocks a sequence can gain over the timed steps
    N = int(sum(-(-int(n) // B) for n in lens) + grow * S + 64)
    order = np.random.default_rng(322).permutation(N)
    width = int(max(-(-int(n) // B) for n in lens)) + grow

    def setup(cls):
        bm = cls(N, B, order)
        for s, n in enumerate(lens):
            bm.add_seq(s)
            bm.append(s, int(n))
        return bm

    cpp, model = setup(BlockManager), setup(BlockManagerModel)
    seqs = np.arange(S, dtype=np.int64)

    t0 = time.perf_counter()
    for _ in range(steps):
        cpp.append_batch(seqs)
        cpp.block_tables_array(seqs, width)
    cpp_step_us = (time.perf_counter() - t0) / steps * 1e6
    msteps = max(3, steps // 10)
    t0 = time.perf_counter()
    for _ in range(msteps):
        for s in range(S):
            model.append(s, 1)
        model.block_tables(list(range(S)), width)
    model_step_us = (time.perf_counter() - t0) / msteps * 1e6

    rng = np.random.default_rng(7)
    system = rng.integers(0, 32000, 512).tolist()
    prompts = [system + rng.integers(0, 32000, 64).tolist() for _ in range(256)]

    def admit(cls):
        bm = cls(256 * 40 + 64, B, prefix_cache=True)
        t0 = time.perf_counter()
        for i, p in enumerate(prompts):
            c = bm.add_seq(i, p)
            bm.append(i, len(p) - c, p[c:])
        return (time.perf_counter() - t0) / len(prompts) * 1e6, bm

    cpp_admit_us, cbm = admit(BlockManager)
    model_admit_us, _ = admit(BlockManagerModel)
    reused = sum(1 for b in range(cbm.num_blocks) if cbm.ref_count(b) == 256)
    log(f"decode-step bookkeeping: C++ {cpp_step_us:.1f} us, Python model {model_step_us:.1f} us; "
        f"admission: C++ {cpp_admit_us:.1f} us/prompt, model {model_admit_us:.1f} us/prompt; "
        f"{reused} blocks shared by all 256 prompts")
    result = {
        "metric": "block manager: host microseconds of decode-step bookkeeping (256 sequences)",
        "value": round(cpp_step_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 0,
        "ms_per_step": round(cpp_step_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": WORKLOADS["block-manager"], "num_seqs": S, "block_size": B, "num_blocks": N,
                   "table_width": width},
        "admission_us_per_prompt": round(cpp_admit_us, 2),
        "prefix_blocks_shared_by_all": reused,
        "roofline": None,
        "note": "host-side bookkeeping (no GPU kernel); for scale, the OPT-13B-shaped batch's decode kernel takes ~355 us per step",
        "cpu_baseline": {"value": round(model_step_us, 2), "unit": "us/step", "cores": 1, "kind": "oracle",
                         "sample": f"the Python reference model on the same decode step ({msteps} steps) and "
                                   f"admissions ({model_admit_us:.1f} us/prompt)"},
    }
    print(json.dumps(result), flush=True)


def bench_swap(args, case, pa, torch, dev):
    """Preemption by swapping: the blocks of 16 of the LLaMA-7B-shaped batch's 64 sequences
    move to a pinned host pool (swap-out) and back under new device ids
    (swap-in), one pa_swap_blocks launch each.  Reference: one DMA copy of
    the same number of bytes between a contiguous device buffer and pinned
    host memory (torch's copy_, the runtime's copy engine)."""
    S, H, D, B = case.num_seqs, case.num_heads, case.head_dim, case.block_size
    preempt = list(range(0, S, 4))  # every fourth sequence: 16 of 64
    ids = []
    for s in preempt:
        nb = -(-int(case.context_lens[s]) // B)
        ids.extend(int(b) for b in case.block_tables[s, :nb])
    n = len(ids)
    used = set(int(b) for b in case.block_tables.ravel() if b >= 0)
    free = [b for b in range(case.num_blocks) if b not in used]
    assert len(free) >= n
    kc = torch.from_numpy(case.k_cache).to(dev)
    vc = torch.from_numpy(case.v_cache).to(dev)
    hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_pairs = torch.from_numpy(np.array([[b, i] for i, b in enumerate(ids)], dtype=np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.array([[i, f] for i, f in enumerate(free[:n])], dtype=np.int64)).to(dev)
    block_bytes = H * B * D * case.elem_bytes
    moved = 2 * n * block_bytes  # K and V, each direction
    torch.cuda.synchronize()

    def timed(fn, reps):
        for _ in range(max(1, args.warmup // 5)):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(3, args.steps // 5)
    log(f"swap {n} blocks ({moved / 1e6:.1f} MB) out and in, {reps} repetitions each")
    out_ms = timed(lambda: pa.swap_blocks(hk, hv, kc, vc, out_pairs), reps)
    in_ms = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, in_pairs), reps)
    # Copy-engine reference: contiguous buffers of the same size.
    dbuf = torch.empty(moved // 2, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(moved // 2, dtype=torch.uint8, pin_memory=True)
    d2h_ms = timed(lambda: (hbuf.copy_(dbuf, non_blocking=True), hbuf.copy_(dbuf, non_blocking=True)), reps)
    h2d_ms = timed(lambda: (dbuf.copy_(hbuf, non_blocking=True), dbuf.copy_(hbuf, non_blocking=True)), reps)
    # Check the round trip once (bitwise) outside the timed region.
    pa.swap_blocks(hk, hv, kc, vc, out_pairs)
    pa.swap_blocks(kc, vc, hk, hv, in_pairs)
    torch.cuda.synchronize()
    src = torch.tensor(ids, device=dev)
    dst = torch.tensor(free[:n], device=dev)
    ok = bool(torch.equal(kc[dst].view(torch.int16), kc[src].view(torch.int16))
              and torch.equal(vc[dst].view(torch.int16), vc[src].view(torch.int16)))
    gbs = lambda ms: round(moved / (ms * 1e-3) / 1e9, 2)
    step_ms = out_ms + in_ms
    log(f"swap-out {out_ms*1e3:.1f} us ({gbs(out_ms)} GB/s), swap-in {in_ms*1e3:.1f} us ({gbs(in_ms)} GB/s); "
        f"DMA reference D2H {gbs(d2h_ms)} GB/s, H2D {gbs(h2d_ms)} GB/s; round trip {'ok' if ok else 'MISMATCH'}")
    result = {
        "metric": "KV block swapping: host-link GB/s per direction",
        "value": round(2 * moved / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": max(1, args.warmup // 5),
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": SWAP_WORKLOAD, "step": "pa_swap_blocks out (device -> pinned host) + in (host -> "
                   "device)", "blocks": n, "block_bytes": block_bytes, "bytes_each_way": moved},
        "swap_out_GBps": gbs(out_ms),
        "swap_in_GBps": gbs(in_ms),
        "dma_reference": {"d2h_GBps": gbs(d2h_ms), "h2d_GBps": gbs(h2d_ms),
                          "what": "torch copy_ of one contiguous buffer of the same size (copy engine)"},
        "round_trip_bitwise_ok": ok,
        "roofline": {
            "kernel": "pa_swap_blocks (copy_pool_blocks_kernel), event-timed, out and in",
            "bound": "link",
            "achieved": round(2 * moved / (step_ms * 1e-3) / 1e9, 2),
            "peak": LINK_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(2 * moved / (step_ms * 1e-3) / 1e9 / LINK_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": int(moved),
        },
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
