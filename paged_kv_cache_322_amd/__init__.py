"""Paged decode and prefill attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libpa.so`` (C ABI declared in ``include/pa.h``).
The functions here only check tensor shapes and types, turn torch tensors
into device pointers plus the current HIP stream, and call the library;
every step of the computation runs in the library's HIP kernels.  PyTorch
supplies device memory and streams only.

If ``libpa.so`` has not been built, importing this package raises
ImportError: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PagedAttentionError",
    "LIB_PATH",
    "lib",
    "decode",
    "append_decode",
    "decode_workspace_size",
    "reshape_and_cache",
    "copy_blocks",
    "status_string",
    "partition_tokens",
    "prefill",
    "swap_blocks",
    "hbm_read_probe",
    "decode_static",
    "STATIC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python paged_kv_cache_322_amd/build.py` "
        "(or __graft_entry__.build()) first"
    )

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

lib.pa_status_string.restype = ctypes.c_char_p
lib.pa_status_string.argtypes = [ctypes.c_int]
lib.pa_decode_partition_tokens.restype = _i32
lib.pa_decode_partition_tokens.argtypes = [_i32, _i32, _i32, _i32, _i32]
lib.pa_decode_workspace_size.restype = ctypes.c_size_t
lib.pa_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
lib.pa_decode.restype = ctypes.c_int
_u32 = ctypes.c_uint32
lib.pa_decode.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                          ctypes.c_float, _i32, _i32, _u32, _p, ctypes.c_size_t, _p]
lib.pa_append_decode.restype = ctypes.c_int
lib.pa_append_decode.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i64, ctypes.c_float, _i32, _i32, _u32, _p, ctypes.c_size_t, _p]
lib.pa_reshape_and_cache.restype = ctypes.c_int
lib.pa_reshape_and_cache.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _p]
lib.pa_copy_blocks.restype = ctypes.c_int
lib.pa_copy_blocks.argtypes = [_p, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _p]
lib.pa_swap_blocks.restype = ctypes.c_int
lib.pa_swap_blocks.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i64, _i64, _i32, _p]
lib.pa_prefill.restype = ctypes.c_int
lib.pa_prefill.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           _i64, ctypes.c_float, _i32, _p]

lib.pa_decode_static.restype = ctypes.c_int
lib.pa_decode_static.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                 ctypes.c_float, _i32, _i32, _u32, _p]
STATIC_SCRATCH_BYTES = 32 << 20  # PA_STATIC_SCRATCH_BYTES
lib.pa_hbm_read_probe.restype = ctypes.c_int
lib.pa_hbm_read_probe.argtypes = [_p, ctypes.c_size_t, _p, _i32, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_uint32, _p]

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
SHARED_BLOCKS = 1  # PA_DECODE_SHARED_BLOCKS


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}")
        self.status = status


def status_string(status: int) -> str:
    return lib.pa_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PagedAttentionError(status, what)


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _code(dtype: torch.dtype) -> int:
    try:
        return _DTYPE_CODE[dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {dtype}; use float32, float16 or bfloat16") from None


def partition_tokens(num_seqs: int, num_heads: int, max_context_len: int, partition_size: int = 0,
                     num_kv_heads: Optional[int] = None) -> int:
    """KV partition length ``decode`` uses (``partition_size`` 0 = library default;
    ``num_kv_heads`` defaults to ``num_heads``, multi-head attention)."""
    hk = num_heads if num_kv_heads is None else num_kv_heads
    return int(lib.pa_decode_partition_tokens(num_seqs, num_heads, hk, max_context_len, partition_size))


def decode_workspace_size(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                          partition_size: int = 0, num_kv_heads: Optional[int] = None) -> int:
    """Bytes of scratch ``decode`` needs (0 if no sequence spans two partitions)."""
    hk = num_heads if num_kv_heads is None else num_kv_heads
    return int(lib.pa_decode_workspace_size(num_seqs, num_heads, hk, head_dim, max_context_len, partition_size))


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len,
                 partition_size, workspace, stream, allocate=True):
    _dev(query, "query", ndim=3)
    dt = query.dtype
    _dev(out, "out", dt, 3)
    _dev(key_cache, "key_cache", dt, 4)
    _dev(value_cache, "value_cache", dt, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(context_lens, "context_lens", torch.int32, 1)
    S, H, D = query.shape
    N, Hk, B, Dk = key_cache.shape
    if tuple(out.shape) != (S, H, D) or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("out/value_cache shapes do not match query/key_cache")
    if Dk != D or H % Hk:
        raise ValueError(f"key_cache heads/head_dim {Hk}/{Dk} do not fit query {H}/{D} "
                         "(query heads must be a multiple of K/V heads)")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    need = decode_workspace_size(S, H, D, max_context_len, partition_size, Hk) if allocate else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=query.device)
    ws_ptr, ws_bytes = 0, 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    tail = (block_tables.data_ptr(), context_lens.data_ptr(), S, H, Hk, D, B, block_tables.shape[1],
            int(max_context_len), N)
    return dt, tail, ws_ptr, ws_bytes


def decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, max_context_len: int,
           partition_size: int = 0, workspace: Optional[torch.Tensor] = None, stream=None,
           shared_blocks: bool = False, siblings: int = 0) -> torch.Tensor:
    """Paged single-query attention (``pa_decode``); writes and returns ``out``.

    out, query [S, H, D]; key_cache, value_cache [N, Hk, B, D] (Hk divides H:
    grouped-query attention when Hk < H); block_tables
    int32 [S, W]; context_lens int32 [S]; ``max_context_len`` a host bound on
    context_lens.  ``workspace`` (uint8, >= decode_workspace_size bytes) is
    allocated from torch's caching allocator when not given.
    ``shared_blocks``: some blocks are read by several sequences (forked
    samples, shared prefixes): load K/V through the caches.
    ``siblings`` (2 .. 16): consecutive groups of that many sequences are
    forked siblings; their common leading blocks are read once per group
    (``PA_DECODE_SIBLINGS``).
    """
    dt, tail, ws_ptr, ws_bytes = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                                              max_context_len, partition_size, workspace, stream)
    flags = (SHARED_BLOCKS if shared_blocks else 0) | (int(siblings) << 8)
    st = lib.pa_decode(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), *tail,
                       float(scale), _code(dt), int(partition_size), flags, ws_ptr, ws_bytes,
                       _stream_handle(query.device, stream))
    _check(st, "pa_decode")
    return out


def decode_static(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                  block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, max_context_len: int,
                  partition_size: int = 0, stream=None, shared_blocks: bool = False,
                  siblings: int = 0) -> torch.Tensor:
    """``decode`` through ``pa_decode_static``: no workspace, none allocated;
    split-K partials go to the library's static per-GPU scratch
    (``STATIC_SCRATCH_BYTES``).  Calls overlapping on one GPU race on it.
    ``shared_blocks`` and ``siblings`` as for ``decode``."""
    dt, tail, _, _ = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len,
                                  partition_size, None, stream, allocate=False)
    st = lib.pa_decode_static(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                              *tail, float(scale), _code(dt), int(partition_size),
                              (SHARED_BLOCKS if shared_blocks else 0) | (int(siblings) << 8),
                              _stream_handle(query.device, stream))
    _check(st, "pa_decode_static")
    return out


def append_decode(out: torch.Tensor, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                  key_cache: torch.Tensor, value_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, scale: float, max_context_len: int, partition_size: int = 0,
                  workspace: Optional[torch.Tensor] = None, stream=None, shared_blocks: bool = False) -> torch.Tensor:
    """One decode step (``pa_append_decode``): store key/value [S, Hk, D] as the
    newest token (position context_lens[s] - 1) of every sequence, then
    attend; writes the caches and ``out``, returns ``out``."""
    dt, tail, ws_ptr, ws_bytes = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                                              max_context_len, partition_size, workspace, stream)
    _dev(key, "key", dt, 3)
    _dev(value, "value", dt, 3)
    kv_shape = (query.shape[0], key_cache.shape[1], query.shape[2])
    if tuple(key.shape) != kv_shape or tuple(value.shape) != kv_shape:
        raise ValueError(f"key/value must have shape [S, Hk, D] = {kv_shape}")
    st = lib.pa_append_decode(out.data_ptr(), query.data_ptr(), key.data_ptr(), value.data_ptr(),
                              key_cache.data_ptr(), value_cache.data_ptr(), *tail, float(scale), _code(dt),
                              int(partition_size), SHARED_BLOCKS if shared_blocks else 0, ws_ptr, ws_bytes,
                              _stream_handle(query.device, stream))
    _check(st, "pa_append_decode")
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write key/value [T, H, D] into the slots named by ``slot_mapping`` (int64 [T])."""
    _dev(key, "key", ndim=3)
    dt = key.dtype
    _dev(value, "value", dt, 3)
    _dev(key_cache, "key_cache", dt, 4)
    _dev(value_cache, "value_cache", dt, 4)
    _dev(slot_mapping, "slot_mapping", torch.int64, 1)
    T, H, D = key.shape
    N, Hk, B, Dk = key_cache.shape
    if tuple(value.shape) != (T, H, D) or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("value/value_cache shapes do not match key/key_cache")
    if Hk != H or Dk != D or slot_mapping.shape[0] != T:
        raise ValueError("key, caches and slot_mapping disagree on tokens/heads/head_dim")
    st = lib.pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        slot_mapping.data_ptr(), T, H, D, B, N, _code(dt), _stream_handle(key.device, stream),
    )
    _check(st, "pa_reshape_and_cache")


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_pairs: torch.Tensor,
                stream=None) -> None:
    """Copy whole blocks: cache[dst] = cache[src] for each (src, dst) row of int64 ``block_pairs``."""
    _dev(key_cache, "key_cache", ndim=4)
    dt = key_cache.dtype
    _dev(value_cache, "value_cache", dt, 4)
    _dev(block_pairs, "block_pairs", torch.int64)
    if block_pairs.numel() % 2:
        raise ValueError("block_pairs must have shape [n, 2]")
    N, H, B, D = key_cache.shape
    if tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("value_cache shape differs from key_cache")
    st = lib.pa_copy_blocks(
        key_cache.data_ptr(), value_cache.data_ptr(), block_pairs.data_ptr(), block_pairs.numel() // 2,
        H, D, B, N, _code(dt), _stream_handle(key_cache.device, stream),
    )
    _check(st, "pa_copy_blocks")


def prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor, scale: float,
            max_query_len: int, max_context_len: int, stream=None) -> torch.Tensor:
    """Causal attention of packed query chunks over the paged context (``pa_prefill``).

    out, query [T, H, D] (f16/bf16, D in {64, 128, 256}); key_cache, value_cache
    [N, Hk, B, D] with the chunks' K/V already written; block_tables int32
    [S, W]; context_lens int32 [S] (chunks included); query_start int32
    [S + 1] (sequence s owns query rows query_start[s] .. query_start[s+1]-1,
    at positions ctx - n .. ctx - 1); host bounds ``max_query_len`` and
    ``max_context_len``.  Writes and returns ``out``.
    """
    _dev(query, "query", ndim=3)
    dt = query.dtype
    _dev(out, "out", dt, 3)
    _dev(key_cache, "key_cache", dt, 4)
    _dev(value_cache, "value_cache", dt, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(context_lens, "context_lens", torch.int32, 1)
    _dev(query_start, "query_start", torch.int32, 1)
    T, H, D = query.shape
    N, Hk, B, Dk = key_cache.shape
    S = context_lens.shape[0]
    if tuple(out.shape) != (T, H, D) or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("out/value_cache shapes do not match query/key_cache")
    if Dk != D or H % Hk:
        raise ValueError(f"key_cache heads/head_dim {Hk}/{Dk} do not fit query {H}/{D}")
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables needs one row and query_start S + 1 entries for S sequences")
    st = lib.pa_prefill(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                        block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), S, T, H, Hk, D,
                        B, block_tables.shape[1], int(max_query_len), int(max_context_len), N, float(scale),
                        _code(dt), _stream_handle(query.device, stream))
    _check(st, "pa_prefill")
    return out


def _pool(t: torch.Tensor, name: str, dtype=None, ndim=None) -> None:
    """A tensor the library may dereference on the device: on the GPU, or in
    pinned (page-locked, mapped) host memory."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type == "cpu" and not t.is_pinned():
        raise ValueError(f"{name} is pageable host memory; allocate it with pin_memory=True")
    if t.device.type not in ("cpu", "cuda"):
        raise ValueError(f"{name} must be on a GPU or in pinned host memory, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def swap_blocks(dst_k: torch.Tensor, dst_v: torch.Tensor, src_k: torch.Tensor, src_v: torch.Tensor,
                block_pairs: torch.Tensor, stream=None) -> None:
    """Move whole blocks between two pools (``pa_swap_blocks``): dst[d] = src[s]
    for each (s, d) row of int64 ``block_pairs``.  Pools are [N, H, B, D] on the
    GPU or in pinned host memory (swap-out: GPU -> host; swap-in: host -> GPU);
    the launch goes on ``stream`` (default: the current stream of the GPU)."""
    _pool(src_k, "src_k", ndim=4)
    dt = src_k.dtype
    _pool(src_v, "src_v", dt, 4)
    _pool(dst_k, "dst_k", dt, 4)
    _pool(dst_v, "dst_v", dt, 4)
    _pool(block_pairs, "block_pairs", torch.int64)
    if block_pairs.numel() % 2:
        raise ValueError("block_pairs must have shape [n, 2]")
    Ns, H, B, D = src_k.shape
    Nd = dst_k.shape[0]
    if tuple(src_v.shape) != tuple(src_k.shape) or tuple(dst_v.shape) != tuple(dst_k.shape):
        raise ValueError("K and V pools of one side differ in shape")
    if tuple(dst_k.shape[1:]) != (H, B, D):
        raise ValueError("the pools disagree on heads, block size or head_dim")
    dev = next((t.device for t in (dst_k, src_k) if t.device.type == "cuda"), torch.device("cuda"))
    st = lib.pa_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), src_k.data_ptr(), src_v.data_ptr(),
                            block_pairs.data_ptr(), block_pairs.numel() // 2, H, D, B, Ns, Nd, _code(dt),
                            _stream_handle(dev, stream))
    _check(st, "pa_swap_blocks")


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, num_workgroups: int, nontemporal: bool = True,
                   run_bytes: int = 0, magic: int = 0x5A17C0DE, stream=None, scattered: bool = False) -> None:
    """Read every byte of ``buf`` once (``pa_hbm_read_probe``, a measurement
    aid): the achievable streaming-read rate.  ``run_bytes`` 0 strides the
    workgroups over the whole buffer; a multiple of 8192 gives each workgroup
    whole contiguous runs of that size (``scattered``: visited in a scattered
    order, as paged blocks lie in the pool).  ``sink`` is a uint32-sized device
    tensor of ``num_workgroups`` elements, written only where a workgroup's
    data XOR to ``magic``."""
    _dev(buf, "buf")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < 4 * num_workgroups:
        raise ValueError("sink must hold num_workgroups uint32 values")
    st = lib.pa_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                               int(num_workgroups), int(run_bytes), int(magic) & 0xFFFFFFFF,
                               (1 if nontemporal else 0) | (2 if scattered else 0),
                               _stream_handle(buf.device, stream))
    _check(st, "pa_hbm_read_probe")
