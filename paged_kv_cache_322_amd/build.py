"""Build libpa.so (the gfx950 HIP kernels and their C ABI) in place.

    python paged_kv_cache_322_amd/build.py

(Run it as a script: importing the package loads the existing libpa.so.)

Compiles every source under ``csrc/`` with hipcc for gfx950 and links them
into ``libpa.so`` next to this file.  Always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa.so")
OBJDIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["pa_decode.hip", "pa_decode_f32.hip", "pa_decode_f16.hip", "pa_decode_bf16.hip", "pa_prefill.hip",
           "pa_cache.hip", "pa_api.hip", "pa_probe.hip", "pa_block_manager.cpp"]

# Host-only C++ (the block manager): built by the host compiler.
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror", f"-I{os.path.join(ROOT, 'include')}"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Werror",
    # Keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions.
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libpa.so")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, src + ".o")
        if src.endswith(".cpp"):
            cmd = [shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        else:
            cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
