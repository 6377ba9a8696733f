"""Python binding of ``libpa.so``: paged decode attention for MI355X (gfx950).

The binding only marshals arguments: it turns torch device tensors into pointers and sizes,
passes torch's current HIP stream, and turns a non-zero status into :class:`PaError`. Every
step of the computation runs in the library's HIP kernels; there is no fallback. Importing
this package fails if ``libpa.so`` has not been built (``python paged_kv_cache_287_amd/build.py``).

torch is imported first so that its HIP runtime (``libamdhip64.so.7``) is the one the library
binds to: the library is linked without an RPATH and resolves that SONAME to the copy already
in the process, so torch's stream handles and device pointers are valid inside it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_WORKSPACE", "PA_ERR_HIP",
    "PA_KV_F16", "PA_KV_FP8_E4M3", "PaError", "LIB_PATH", "lib", "EXPORTED_SYMBOLS",
    "decode_workspace_bytes", "decode_workspace_reset", "decode_partition_tokens", "pa_decode",
    "pa_decode_append", "pa_decode_append_noalloc", "NOALLOC_SCRATCH_BYTES",
    "shared_prefix_workspace_bytes", "pa_decode_shared_prefix", "pa_decode_shared_prefix_append",
    "pa_prefill", "pa_kv_write",
    "pa_copy_blocks", "pa_swap_blocks", "stream_read_probe",
]

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
PA_KV_F16, PA_KV_FP8_E4M3 = 0, 1
ABI_VERSION = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")

_p, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float

#: every entry point declared in include/pa.h with its (restype, argtypes)
EXPORTED_SYMBOLS = {
    "pa_abi_version": (ctypes.c_int, []),
    "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_hip_error": (ctypes.c_int, []),
    "pa_decode_partition_tokens": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "pa_decode_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                        _i32, _p, _sz, _p]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_shared_prefix": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "pa_decode_shared_prefix_append": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                      _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                                      _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      _f32, _i32, _p, _sz, _p]),
    "pa_prefill": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p]),
    "pa_kv_write": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _p]),
    "pa_copy_blocks": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p]),
    "pa_swap_blocks": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _p]),
    "pa_stream_read_probe": (ctypes.c_int, [_p, _sz, _p, _p]),
    "pa_decode_workspace_reset": (ctypes.c_int, [_p, _sz, _p]),
    "pa_decode_append_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _i32, _f32, _i32, _p]),
}

#: bytes of the library's own per-GPU decode workspace (pa_decode_append_noalloc)
NOALLOC_SCRATCH_BYTES = 16 << 20


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.pa_status_str(status).decode()
        if status == PA_ERR_HIP:
            msg += f" (hipError_t {lib.pa_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_287_amd/build.py`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTED_SYMBOLS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    if handle.pa_abi_version() != ABI_VERSION:
        raise ImportError(f"libpa.so ABI {handle.pa_abi_version()} != binding ABI {ABI_VERSION}")
    return handle


lib = _load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# The checks and the stream lookup below run on every call, so they are kept cheap: a decode
# call of a small batch runs for 15-20 us on the GPU, and the host spent ~15 us per call when
# it looked up torch.cuda.current_stream() (~2.8 us) and tested each tensor attribute apart.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> Optional[int]:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if (isinstance(t, torch.Tensor) and t.dtype in dtypes and t.dim() == ndim and t.is_cuda
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    raise ValueError(f"{name} must be a device tensor")


def _check_order(seq_order: Optional[torch.Tensor], num_seqs: int) -> None:
    if seq_order is None:
        return
    _check(seq_order, "seq_order", (torch.int32,), 1)
    if seq_order.shape[0] != num_seqs:
        raise ValueError("seq_order must have one entry per sequence")


def _kv_dtype(cache: torch.Tensor) -> int:
    if cache.dtype == torch.float16:
        return PA_KV_F16
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_KV_FP8_E4M3
    raise TypeError(f"KV cache dtype {cache.dtype} is not supported")


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           block_size: int, max_context_len: int, kv_dtype: int = PA_KV_F16,
                           partition_tokens: int = 0) -> int:
    """Workspace bytes for pa_decode (allocate zero-filled: it holds counters)."""
    return int(lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size, max_context_len, kv_dtype, partition_tokens))


def decode_workspace_reset(workspace: torch.Tensor, *, stream=None) -> None:
    """Enqueue a clear of the workspace's counter zone (fresh memory, or recovery after a call
    that did not complete)."""
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    st = lib.pa_decode_workspace_reset(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_workspace_reset")


def decode_partition_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            block_size: int, max_context_len: int, kv_dtype: int = PA_KV_F16,
                            partition_tokens: int = 0) -> int:
    return int(lib.pa_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, kv_dtype, partition_tokens))


def pa_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, *,
              k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
              max_context_len: int = 0, partition_tokens: int = 0,
              workspace: Optional[torch.Tensor] = None, seq_order: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Enqueue paged decode attention; writes ``out`` [S, Hq, D] fp16 and returns it.

    ``seq_order`` (optional int32 device tensor [S], a permutation) is the dispatch order of the
    sequences, e.g. longest first; ``out`` stays in batch order.

    ``workspace`` (uint8 device tensor, zero-filled before its first use) is allocated here,
    zero-filled, when omitted and needed.
    """
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_seqs, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    mbps = block_tables.shape[1]
    if workspace is None:
        need = decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_context_len if max_context_len > 0 else mbps * block_size,
                                      kvt, partition_tokens)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check_order(seq_order, num_seqs)
    st = lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                       _ptr(block_tables), _ptr(context_lens), _ptr(seq_order), num_seqs, num_q_heads, num_kv_heads,
                       head_dim, block_size, nb, mbps, max_context_len, partition_tokens,
                       float(scale), kvt,
                       _ptr(workspace), ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode")
    return out


def pa_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, *,
                     k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                     max_context_len: int = 0, partition_tokens: int = 0,
                     workspace: Optional[torch.Tensor] = None,
                     seq_order: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Enqueue one decode step: store each sequence's new K/V row ``k_new/v_new[b]`` at
    ``slot_mapping[b]`` and attend over the cache including it; writes ``out`` and returns it.

    Equal, bit for bit, to ``pa_kv_write`` of the S new rows followed by ``pa_decode``.
    ``workspace`` as for ``pa_decode``.
    """
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_new, "k_new", (torch.float16,), 3)
    _check(v_new, "v_new", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(slot_mapping, "slot_mapping", (torch.int64,), 1)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_seqs, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if k_new.shape != (num_seqs, num_kv_heads, head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [num_seqs, Hkv, head_dim]")
    if (block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs
            or slot_mapping.shape[0] != num_seqs):
        raise ValueError("block_tables / context_lens / slot_mapping must have one row per sequence")
    mbps = block_tables.shape[1]
    if workspace is None:
        need = decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_context_len if max_context_len > 0 else mbps * block_size,
                                      kvt, partition_tokens)
        if need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check_order(seq_order, num_seqs)
    st = lib.pa_decode_append(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                              _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping),
                              _ptr(block_tables), _ptr(context_lens), _ptr(seq_order), num_seqs,
                              num_q_heads,
                              num_kv_heads, head_dim, block_size, nb, mbps, max_context_len,
                              partition_tokens, float(scale), kvt, _ptr(workspace), ws_bytes,
                              _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_append")
    return out


def pa_decode_append_noalloc(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                             v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             slot_mapping: torch.Tensor, block_tables: torch.Tensor,
                             context_lens: torch.Tensor, scale: float, *,
                             k_scale: Optional[torch.Tensor] = None,
                             v_scale: Optional[torch.Tensor] = None, max_context_len: int = 0,
                             partition_tokens: int = 0, seq_order: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """``pa_decode_append`` whose workspace is the library's own per-GPU device array: neither
    this binding nor the library allocates. Calls that overlap on one GPU race on that array."""
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_new, "k_new", (torch.float16,), 3)
    _check(v_new, "v_new", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(slot_mapping, "slot_mapping", (torch.int64,), 1)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_seqs, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if k_new.shape != (num_seqs, num_kv_heads, head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [num_seqs, Hkv, head_dim]")
    if (block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs
            or slot_mapping.shape[0] != num_seqs):
        raise ValueError("block_tables / context_lens / slot_mapping must have one row per sequence")
    _check_order(seq_order, num_seqs)
    st = lib.pa_decode_append_noalloc(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                      _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens),
                                      _ptr(seq_order), num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, nb,
                                      block_tables.shape[1], max_context_len, partition_tokens,
                                      float(scale), kvt, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_append_noalloc")
    return out


def shared_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                  head_dim: int, block_size: int, max_context_len: int,
                                  kv_dtype: int = PA_KV_F16, partition_tokens: int = 0) -> int:
    """Workspace bytes for pa_decode_shared_prefix (allocate zero-filled: it holds counters)."""
    return int(lib.pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                           head_dim, block_size, max_context_len,
                                                           kv_dtype, partition_tokens))


def pa_decode_shared_prefix(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, group_start: torch.Tensor,
                            group_prefix_blocks: torch.Tensor, scale: float, *,
                            max_group_seqs: int, max_prefix_blocks: int, k_scale: Optional[torch.Tensor] = None,
                            v_scale: Optional[torch.Tensor] = None, max_context_len: int = 0,
                            partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
                            seq_order: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Enqueue decode attention whose shared prefix blocks are read once per group and KV head;
    writes ``out`` [S, Hq, D] fp16 and returns it.

    ``group_start`` [NG + 1] and ``group_prefix_blocks`` [NG] are int32 device tensors;
    ``max_group_seqs`` and ``max_prefix_blocks`` (host) bound every group's size and prefix.
    """
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    _check(group_start, "group_start", (torch.int32,), 1)
    _check(group_prefix_blocks, "group_prefix_blocks", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_seqs, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    num_groups = group_prefix_blocks.shape[0]
    if group_start.shape[0] != num_groups + 1:
        raise ValueError("group_start must have one entry per group plus one")
    mbps = block_tables.shape[1]
    if workspace is None:
        need = shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size,
                                             max_context_len if max_context_len > 0 else mbps * block_size,
                                             kvt, partition_tokens)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check_order(seq_order, num_seqs)
    st = lib.pa_decode_shared_prefix(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
                                     _ptr(seq_order), _ptr(group_start), _ptr(group_prefix_blocks), num_groups,
                                     int(max_group_seqs), int(max_prefix_blocks), num_seqs, num_q_heads, num_kv_heads,
                                     head_dim, block_size, nb, mbps, max_context_len,
                                     partition_tokens, float(scale), kvt, _ptr(workspace),
                                     ws_bytes, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_shared_prefix")
    return out


def pa_decode_shared_prefix_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                   v_new: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor,
                                   group_start: torch.Tensor, group_prefix_blocks: torch.Tensor,
                                   scale: float, *, max_group_seqs: int, max_prefix_blocks: int,
                                   k_scale: Optional[torch.Tensor] = None,
                                   v_scale: Optional[torch.Tensor] = None,
                                   max_context_len: int = 0, partition_tokens: int = 0,
                                   workspace: Optional[torch.Tensor] = None,
                                   seq_order: Optional[torch.Tensor] = None,
                                   stream=None) -> torch.Tensor:
    """Enqueue one decode step for a batch with shared prefixes: store each sequence's new K/V
    row at ``slot_mapping[b]`` and decode as ``pa_decode_shared_prefix``; equal, bit for bit, to
    ``pa_kv_write`` of the new rows followed by ``pa_decode_shared_prefix``."""
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_new, "k_new", (torch.float16,), 3)
    _check(v_new, "v_new", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(slot_mapping, "slot_mapping", (torch.int64,), 1)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    _check(group_start, "group_start", (torch.int32,), 1)
    _check(group_prefix_blocks, "group_prefix_blocks", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_seqs, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if k_new.shape != (num_seqs, num_kv_heads, head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [num_seqs, Hkv, head_dim]")
    if (block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs
            or slot_mapping.shape[0] != num_seqs):
        raise ValueError("block_tables / context_lens / slot_mapping must have one row per sequence")
    num_groups = group_prefix_blocks.shape[0]
    if group_start.shape[0] != num_groups + 1:
        raise ValueError("group_start must have one entry per group plus one")
    _check_order(seq_order, num_seqs)
    mbps = block_tables.shape[1]
    if workspace is None:
        need = shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size,
                                             max_context_len if max_context_len > 0 else mbps * block_size,
                                             kvt, partition_tokens)
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.pa_decode_shared_prefix_append(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), _ptr(seq_order),
        _ptr(group_start), _ptr(group_prefix_blocks), num_groups, int(max_group_seqs),
        int(max_prefix_blocks), num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, nb, mbps,
        max_context_len, partition_tokens, float(scale), kvt, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_decode_shared_prefix_append")
    return out


def pa_prefill(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
               scale: float, *, max_query_len: int, max_context_len: int = 0,
               k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """Enqueue causal chunk attention over the paged cache; writes ``out`` [T, Hq, D] fp16.

    ``query_start`` [S + 1] int32 (device) gives each sequence's first row in ``q`` / ``out``;
    ``max_query_len`` bounds every chunk length and ``max_context_len`` (0 = the table's width
    times the block size) every context length; both are host integers that size the grid.
    """
    _check(q, "q", (torch.float16,), 3)
    _check(out, "out", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(block_tables, "block_tables", (torch.int32,), 2)
    _check(context_lens, "context_lens", (torch.int32,), 1)
    _check(query_start, "query_start", (torch.int32,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    num_tokens, num_q_heads, head_dim = q.shape
    nb, num_kv_heads, block_size, d2 = k_cache.shape
    num_seqs = context_lens.shape[0]
    if out.shape != q.shape or d2 != head_dim or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between q, out and the caches")
    if block_tables.shape[0] != num_seqs or query_start.shape[0] != num_seqs + 1:
        raise ValueError("block_tables needs one row and query_start one entry per sequence (+1)")
    mbps = block_tables.shape[1]
    st = lib.pa_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                        _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), _ptr(query_start),
                        num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size, nb,
                        mbps, int(max_query_len),
                        int(max_context_len) if max_context_len > 0 else mbps * block_size,
                        float(scale), kvt, _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_prefill")
    return out


def pa_kv_write(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                slot_mapping: torch.Tensor, *, k_scale: Optional[torch.Tensor] = None,
                v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue the slot-mapped append of new K/V rows [T, Hkv, D] into the caches (E4M3 caches
    need their per-(block, head) scales, which the append updates)."""
    _check(k, "k", (torch.float16,), 3)
    _check(v, "v", (torch.float16,), 3)
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(slot_mapping, "slot_mapping", (torch.int64,), 1)
    kvt = _kv_dtype(k_cache)
    if kvt == PA_KV_FP8_E4M3:
        for n, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is None:
                raise ValueError(f"{n} is required for an 8-bit cache")
            _check(s, n, (torch.float32,), 2)
    nb, hkv, bs, d = k_cache.shape
    if k.shape != v.shape or k.shape[1:] != (hkv, d) or slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("shape mismatch between k, v, slot_mapping and the caches")
    st = lib.pa_kv_write(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                         _ptr(v_scale), _ptr(slot_mapping), k.shape[0], hkv, d, bs, nb, kvt,
                         _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_kv_write")


def pa_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor, *,
                   k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Enqueue copy-on-write block copies for every (src, dst) row of ``block_mapping`` [P, 2]."""
    _check(k_cache, "k_cache", (torch.float16, torch.uint8, torch.float8_e4m3fn), 4)
    _check(v_cache, "v_cache", (k_cache.dtype,), 4)
    _check(block_mapping, "block_mapping", (torch.int32,), 2)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [P, 2]")
    nb, hkv, bs, d = k_cache.shape
    st = lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                            _ptr(block_mapping), block_mapping.shape[0], hkv, d, bs, nb,
                            _kv_dtype(k_cache), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_copy_blocks")


def pa_swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor,
                   dst_v: torch.Tensor, block_mapping: torch.Tensor, *,
                   src_k_scale: Optional[torch.Tensor] = None, src_v_scale: Optional[torch.Tensor] = None,
                   dst_k_scale: Optional[torch.Tensor] = None, dst_v_scale: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    """Enqueue whole-block copies between two pools [NB, Hkv, BS, D] (device tensors, or pinned
    host tensors made with ``pin_memory=True``) for every (src, dst) row of ``block_mapping``."""
    for n, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous [NB, Hkv, BS, D] tensor")
        if t.device.type != "cuda" and not t.is_pinned():
            raise ValueError(f"{n} must be device memory or pinned host memory")
        if t.dtype != src_k.dtype:
            raise TypeError("all pools must share one dtype")
    _check(block_mapping, "block_mapping", (torch.int32,), 2)
    nb_s, hkv, bs, d = src_k.shape
    nb_d = dst_k.shape[0]
    if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape or dst_k.shape[1:] != src_k.shape[1:]:
        raise ValueError("pool shapes differ")
    st = lib.pa_swap_blocks(_ptr(src_k), _ptr(src_v), _ptr(src_k_scale), _ptr(src_v_scale),
                            _ptr(dst_k), _ptr(dst_v), _ptr(dst_k_scale), _ptr(dst_v_scale),
                            _ptr(block_mapping), block_mapping.shape[0], hkv, d, bs, nb_s, nb_d,
                            _kv_dtype(src_k), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_swap_blocks")


def stream_read_probe(buf: torch.Tensor, sink: torch.Tensor, *, stream=None) -> None:
    """Enqueue one streaming read of ``buf`` (attainable-bandwidth measurement utility)."""
    if buf.device.type != "cuda" or sink.device.type != "cuda":
        raise ValueError("probe buffers must be device tensors")
    st = lib.pa_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream))
    if st != PA_OK:
        raise PaError(st, "pa_stream_read_probe")
