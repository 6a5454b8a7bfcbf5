"""Storage encodings for the synthetic KV workloads.

Values are drawn in float32 and stored in one of three element types:
``f32`` (numpy float32), ``f16`` (numpy float16, IEEE binary16) or ``bf16``
(bfloat16 held as its raw 16-bit pattern in a numpy uint16 array, because
numpy has no bfloat16 type).  Nothing here computes attention; it only turns
float32 draws into stored bits and provides NaN canaries for slots that no
valid token occupies.
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# Element size in bytes of each storage type.
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# Numpy container for each storage type.
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

# Unsigned view used for bitwise comparisons of stored data.
NP_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}

# Quiet-NaN canaries with a recognisable payload.  They fill every pool slot
# that holds no valid token so that a stray read shows up as NaN and a stray
# write shows up as a changed bit pattern.
CANARY_BITS = {"f32": 0x7FC0DEAD, "f16": 0x7E5A, "bf16": 0x7FDA}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    bfloat16 keeps the upper 16 bits of the float32 pattern.  Adding
    0x7FFF plus the lowest kept bit before truncation rounds to nearest with
    ties going to the even pattern.  NaN inputs become the canonical quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    rounded = ((bits + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, np.uint16(0x7FC0), rounded)
    return rounded


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float32 values ``x`` in storage type ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        # numpy's float32 -> float16 cast rounds to nearest even.
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def canary_fill(shape, dtype: str) -> np.ndarray:
    """A storage array of ``shape`` whose every element is the NaN canary."""
    bits = np.full(shape, CANARY_BITS[dtype], dtype=NP_BITS[dtype])
    return bits.view(NP_STORAGE[dtype])


def bits_view(a: np.ndarray) -> np.ndarray:
    """Reinterpret a storage array as unsigned integers of the same width."""
    width = a.dtype.itemsize
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[width])
