"""Shared plumbing for the GPU tests: upload seeded workloads, run the HIP path
through the C ABI binding, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
INT_VIEW = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16}
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def log(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def pa():
    import paged_kv_cache_322_amd as m

    return m


def to_gpu(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def to_storage(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> numpy array in the workloads' storage encoding."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class GpuCase:
    """A workload resident on the GPU."""

    def __init__(self, case: wl.Case):
        self.case = case
        d = case.dtype
        self.q = to_gpu(case.q, d)
        self.kc = to_gpu(case.k_cache, d)
        self.vc = to_gpu(case.v_cache, d)
        self.bt = to_gpu(case.block_tables)
        self.ctx = to_gpu(case.context_lens)
        self.out = torch.empty_like(self.q)
        self.steps = []
        for st in case.steps:
            if isinstance(st, wl.AppendStep):
                self.steps.append(("append", to_gpu(st.key, d), to_gpu(st.value, d), to_gpu(st.slot_mapping)))
            else:
                self.steps.append(("copy", to_gpu(st.pairs)))

    def run_step(self, i: int) -> None:
        st = self.steps[i]
        if st[0] == "append":
            pa().reshape_and_cache(st[1], st[2], self.kc, self.vc, st[3])
        else:
            pa().copy_blocks(self.kc, self.vc, st[1])

    def run_steps(self) -> None:
        for i in range(len(self.steps)):
            self.run_step(i)

    def decode(self, partition: int = 0, out: torch.Tensor | None = None, bt=None, ctx=None, kc=None, vc=None,
               max_context_len=None, shared_blocks: bool = False) -> torch.Tensor:
        out = self.out if out is None else out
        c = self.case
        pa().decode(out, self.q, self.kc if kc is None else kc, self.vc if vc is None else vc,
                    self.bt if bt is None else bt, self.ctx if ctx is None else ctx, c.scale,
                    c.max_context_len if max_context_len is None else max_context_len, partition_size=partition,
                    shared_blocks=shared_blocks)
        return out


def oracle_steps(case: wl.Case):
    """Apply the case's cache updates with the oracle; yields the pools after each."""
    kc, vc = case.k_cache, case.v_cache
    for st in case.steps:
        if isinstance(st, wl.AppendStep):
            kc, vc = oracle.reshape_and_cache(st.key, st.value, kc, vc, st.slot_mapping)
        else:
            kc, vc = oracle.copy_blocks(kc, vc, st.pairs)
        yield kc, vc


def oracle_decode(case: wl.Case, kc, vc, seqs=None) -> np.ndarray:
    idx = np.arange(case.num_seqs) if seqs is None else np.asarray(seqs)
    return oracle.paged_decode(case.q[idx], kc, vc, case.block_tables[idx], case.context_lens[idx], case.scale,
                               case.dtype)


def assert_pool_equal(gpu: torch.Tensor, ref: np.ndarray, dtype: str, what: str) -> None:
    ref_t = to_gpu(ref, dtype)
    iv = INT_VIEW[dtype]
    same = torch.equal(gpu.view(iv), ref_t.view(iv))
    if not same:
        diff = (gpu.view(iv) != ref_t.view(iv)).reshape(gpu.shape[0], -1).any(dim=1).nonzero().flatten()
        raise AssertionError(f"{what}: pool differs from the oracle in blocks {diff[:16].tolist()}")


MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}
MIN_EXP = {"f32": -126, "f16": -14, "bf16": -126}


def out_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output format at |ref| (one unit in the last place)."""
    a = np.maximum(np.abs(ref), np.finfo(np.float64).tiny)
    e = np.maximum(np.floor(np.log2(a)), MIN_EXP[dtype])
    return np.exp2(e - MANT_BITS[dtype])


def assert_close(out: torch.Tensor, ref: np.ndarray, dtype: str, what: str, seqs=None, tol=None,
                 strict: bool = True) -> float:
    """Max-abs check against the float64 oracle.

    strict: |gpu - oracle| <= tol (2e-3 for f16/bf16, 1e-5 for f32).
    not strict: each element may instead be within one ulp of the output
    format at the oracle value.  A correctly rounded result is within half
    an ulp, so this is the tightest bound any implementation that rounds to
    f16/bf16 can meet where |out| is large (bf16 has 8 significant bits:
    half an ulp is 2^-9 ~ 1.95e-3 already on [0.5, 1)).
    """
    got = out.double().cpu().numpy()
    if seqs is not None:
        got = got[np.asarray(seqs)]
    tol = TOL[dtype] if tol is None else tol
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    err = float(diff.max()) if ref.size else 0.0
    if strict:
        log(f"{what}: max |gpu - oracle| = {err:.3e} (tol {tol:g})")
        assert err <= tol, f"{what}: max abs error {err} > {tol}"
    else:
        ulps = float((diff / out_ulp(ref, dtype)).max()) if ref.size else 0.0
        log(f"{what}: max |gpu - oracle| = {err:.3e}, max {ulps:.2f} output ulp (tol {tol:g} or 1 ulp)")
        bad = (diff > tol) & (diff > out_ulp(ref, dtype))
        assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {tol} and beyond one output ulp"
    return err
