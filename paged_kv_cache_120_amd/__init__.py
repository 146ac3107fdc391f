"""Paged KV-cache decode for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/pa.h`` (``libpagedkv.so``,
built in-tree by ``python -m paged_kv_cache_120_amd.build``).  Each function
here has the name of the C entry point it calls and only marshals arguments:
it checks dtypes, devices and contiguity of the torch tensors, then passes
their device pointers and the current HIP stream.  Every step of the path
runs in the library's kernels; there is no fallback: the first call (or
access to ``lib``) raises ImportError if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "PaError", "lib", "library_path", "pa_status_str", "pa_kv_cache_shape",
    "pa_slot_mapping", "pa_cache_write", "pa_copy_blocks", "pa_swap_blocks", "pa_decode",
    "pa_splitk_workspace_size", "pa_decode_splitk", "pa_decode_reduce",
    "pa_balanced_grid", "pa_balanced_workspace_size", "pa_decode_balanced",
    "pa_decode_step", "pa_multi_workspace_size", "pa_decode_multi", "pa_prefill",
    "pa_cache_write_fp8", "pa_balanced_grid_fp8", "pa_decode_balanced_fp8",
    "pa_decode_step_fp8", "pa_multi_balanced_grid", "pa_multi_balanced_workspace_size",
    "pa_multi_balanced_workspace_size_tiles",
    "pa_decode_multi_balanced",
    "pa_prefix_workspace_size", "pa_decode_shared_prefix", "pa_decode_step_noalloc",
    "pa_last_check", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDKV_LIBRARY names another build of the same library (for instance a
# sanitizer build of the host code); the default is the in-tree build
library_path = os.environ.get("PAGEDKV_LIBRARY") or os.path.join(_HERE, "libpagedkv.so")

STATUS = {
    0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
    4: "PA_ERR_ALIGN", 5: "PA_ERR_WORKSPACE", 6: "PA_ERR_HIP", 7: "PA_ERR_CHECK",
}


class PaError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {pa_status_str(status)} ({status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m paged_kv_cache_120_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(library_path)
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "pa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "pa_kv_cache_shape": (None, [i32, i32, i32, i32, ctypes.POINTER(i64)]),
        "pa_slot_mapping": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, i32, i32, vp]),
        "pa_cache_write": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "pa_copy_blocks": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]),
        "pa_swap_blocks": (ctypes.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32,
                                          i32, vp]),
        "pa_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                     i32, i32, f32, vp]),
        "pa_splitk_workspace_size": (sz, [i32, i32, i32, i32, i32, i32]),
        "pa_decode_splitk": (ctypes.c_int, [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                            i32, i32, f32, i32, vp, sz, vp]),
        "pa_decode_reduce": (ctypes.c_int, [vp, vp, sz, vp, i32, i32, i32, i32, i32,
                                            i32, vp]),
        "pa_multi_workspace_size": (sz, [i32, i32, i32, i32, i32, i32]),
        "pa_decode_multi": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i32,
                                           i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]),
        "pa_prefill": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, vp, i32,
                                      i32, i32, i32, i32, i32, f32, vp]),
        "pa_balanced_grid": (i32, [i32, i32, i32, i32]),
        "pa_balanced_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "pa_decode_balanced": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                              i32, i32, i32, f32, i32, vp, sz, vp]),
        "pa_decode_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                          i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]),
        "pa_cache_write_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                              f32, f32, vp]),
        "pa_balanced_grid_fp8": (i32, [i32, i32, i32, i32]),
        "pa_decode_step_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                              i32, i32, i32, i32, i32, i32, f32, f32, f32,
                                              i32, vp, sz, vp]),
        "pa_prefix_workspace_size": (sz, [i32, i32, i32, i32, i32, i32]),
        "pa_multi_balanced_grid": (i32, [i32, i32, i32, i32, i32]),
        "pa_multi_balanced_workspace_size": (sz, [i32, i32, i32, i32]),
        "pa_multi_balanced_workspace_size_tiles": (sz, [i32, i32, i32, i32, i32, i32]),
        "pa_decode_multi_balanced": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                                    vp, i32, i32, i32, i32, i32, i32, f32,
                                                    i32, vp, sz, vp]),
        "pa_decode_shared_prefix": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                                   i32, i32, i32, i32, f32, i32, vp, vp,
                                                   vp, i32, i32, i32, vp, sz, vp]),
        "pa_decode_balanced_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                                  i32, i32, i32, i32, f32, f32, f32, i32,
                                                  vp, sz, vp]),
        "pa_stream_read": (ctypes.c_int, [vp, sz, vp, i32, vp]),
        "pa_last_check": (ctypes.c_uint32, []),
        "pa_decode_step_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                  i32, i32, i32, i32, i32, i32, f32, i32,
                                                  vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def pa_last_check() -> int:
    """PA_CHECK_* bits of the last PA_CHECK=1 validation pass on this thread."""
    return int(_lib().pa_last_check())


def pa_status_str(status: int) -> str:
    return _lib().pa_status_str(int(status)).decode()


def pa_kv_cache_shape(num_blocks: int, block_size: int, num_kv_heads: int,
                      head_size: int) -> Tuple[int, ...]:
    out = (ctypes.c_int64 * 5)()
    _lib().pa_kv_cache_shape(num_blocks, block_size, num_kv_heads, head_size, out)
    return tuple(int(x) for x in out)


def pa_splitk_workspace_size(num_seqs: int, num_heads: int, head_size: int,
                             max_blocks_per_seq: int, block_size: int,
                             partition_size: int) -> int:
    return int(_lib().pa_splitk_workspace_size(num_seqs, num_heads, head_size,
                                            max_blocks_per_seq, block_size,
                                            partition_size))


def pa_balanced_grid(num_heads: int, num_kv_heads: int, head_size: int,
                     block_size: int) -> int:
    """Workgroups of the balanced decode the current device holds at once
    (0 if unknown).  Initialises the HIP runtime on the current device."""
    return int(_lib().pa_balanced_grid(num_heads, num_kv_heads, head_size, block_size))


def pa_balanced_grid_fp8(num_heads: int, num_kv_heads: int, head_size: int,
                         block_size: int) -> int:
    """As pa_balanced_grid, for the decode over an fp8 pool."""
    return int(_lib().pa_balanced_grid_fp8(num_heads, num_kv_heads, head_size,
                                           block_size))


def pa_multi_balanced_grid(num_heads: int, num_kv_heads: int, head_size: int,
                           block_size: int, max_q_per_seq: int) -> int:
    """Resident workgroups of the balanced multi-token kernel for this many
    query rows per sequence (0 if unsupported or unknown)."""
    return int(_lib().pa_multi_balanced_grid(num_heads, num_kv_heads, head_size,
                                             block_size, max_q_per_seq))


def pa_multi_balanced_workspace_size(num_seqs: int, num_kv_heads: int, head_size: int,
                                     grid: int) -> int:
    return int(_lib().pa_multi_balanced_workspace_size(num_seqs, num_kv_heads, head_size,
                                                       grid))


def pa_multi_balanced_workspace_size_tiles(num_seqs: int, num_heads: int,
                                           num_kv_heads: int, head_size: int, grid: int,
                                           max_q_per_seq: int) -> int:
    """Workspace of pa_decode_multi_balanced for any max_q_per_seq (one
    counter and state row group per (sequence, kv head, column tile))."""
    return int(_lib().pa_multi_balanced_workspace_size_tiles(
        num_seqs, num_heads, num_kv_heads, head_size, grid, max_q_per_seq))


def pa_prefix_workspace_size(num_seqs: int, num_heads: int, head_size: int,
                             max_blocks_per_seq: int, block_size: int,
                             partition_size: int) -> int:
    return int(_lib().pa_prefix_workspace_size(num_seqs, num_heads, head_size,
                                               max_blocks_per_seq, block_size,
                                               partition_size))


def pa_balanced_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int,
                               head_size: int, grid: int) -> int:
    return int(_lib().pa_balanced_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                 head_size, grid))


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def _dev(t, dtype, name: str, ndim: Optional[int] = None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _mapped(t, dtype, name: str, ndim: Optional[int] = None) -> int:
    """A device tensor, or a pinned host tensor (its memory is mapped for the
    device at the same address on ROCm)."""
    torch = _torch()
    if isinstance(t, torch.Tensor) and t.device.type == "cpu":
        if not t.is_pinned():
            raise ValueError(f"{name}: a host tensor must be pinned (pin_memory=True)")
        if t.dtype != dtype:
            raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
        return t.data_ptr()
    return _dev(t, dtype, name, ndim)


def _dev_fp8(t, name: str, ndim: int) -> int:
    """An fp8 pool half: uint8 codes or torch.float8_e4m3fn (same bytes)."""
    torch = _torch()
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        return _dev(t, torch.float8_e4m3fn, name, ndim)
    return _dev(t, torch.uint8, name, ndim)


def _check(func: str, status: int) -> None:
    if status != 0:
        raise PaError(func, status)


def pa_slot_mapping(slot_mapping, block_tables, seq_idx, positions,
                    block_size: int, stream=None) -> None:
    """slot_mapping[j] = block_tables[seq_idx[j], positions[j] // B] * B +
    positions[j] % B (int32 device tensors)."""
    torch = _torch()
    n = int(positions.numel())
    _check("pa_slot_mapping", _lib().pa_slot_mapping(
        _dev(slot_mapping, torch.int32, "slot_mapping", 1),
        _dev(block_tables, torch.int32, "block_tables", 2),
        block_tables.shape[1], block_tables.shape[0],
        _dev(seq_idx, torch.int32, "seq_idx", 1),
        _dev(positions, torch.int32, "positions", 1),
        n, block_size, _stream(stream)))


def pa_cache_write(key, value, key_cache, value_cache, slot_mapping,
                   stream=None) -> None:
    """key/value fp16 [N, H_kv, D] -> key_cache/value_cache fp16
    [nb, B, H_kv, D] at slot_mapping (int32 [N])."""
    torch = _torch()
    nb, B, Hkv, D = key_cache.shape
    if tuple(value_cache.shape) != (nb, B, Hkv, D) or key.shape[1:] != (Hkv, D) \
            or value.shape != key.shape:
        raise ValueError("pa_cache_write: inconsistent shapes")
    _check("pa_cache_write", _lib().pa_cache_write(
        _dev(key, torch.float16, "key", 3), _dev(value, torch.float16, "value", 3),
        _dev(key_cache, torch.float16, "key_cache", 4),
        _dev(value_cache, torch.float16, "value_cache", 4),
        _dev(slot_mapping, torch.int32, "slot_mapping", 1),
        key.shape[0], nb, B, Hkv, D, _stream(stream)))


def pa_cache_write_fp8(key, value, key_cache, value_cache, slot_mapping,
                       k_scale: float, v_scale: float, stream=None) -> None:
    """key/value fp16 [N, H_kv, D] -> e4m3 codes of x / scale (clamped to
    +-448) in key_cache/value_cache (uint8 or float8_e4m3fn [nb, B, H_kv, D])
    at slot_mapping (int32 [N])."""
    torch = _torch()
    nb, B, Hkv, D = key_cache.shape
    if tuple(value_cache.shape) != (nb, B, Hkv, D) or key.shape[1:] != (Hkv, D) \
            or value.shape != key.shape:
        raise ValueError("pa_cache_write_fp8: inconsistent shapes")
    _check("pa_cache_write_fp8", _lib().pa_cache_write_fp8(
        _dev(key, torch.float16, "key", 3), _dev(value, torch.float16, "value", 3),
        _dev_fp8(key_cache, "key_cache", 4), _dev_fp8(value_cache, "value_cache", 4),
        _dev(slot_mapping, torch.int32, "slot_mapping", 1),
        key.shape[0], nb, B, Hkv, D, float(k_scale), float(v_scale), _stream(stream)))


def pa_copy_blocks(key_cache, value_cache, src, dst, stream=None) -> None:
    torch = _torch()
    nb, B, Hkv, D = key_cache.shape
    if src.shape != dst.shape:
        raise ValueError("pa_copy_blocks: src/dst shapes differ")
    _check("pa_copy_blocks", _lib().pa_copy_blocks(
        _dev(key_cache, torch.float16, "key_cache", 4),
        _dev(value_cache, torch.float16, "value_cache", 4),
        _dev(src, torch.int32, "src", 1), _dev(dst, torch.int32, "dst", 1),
        src.numel(), nb, B, Hkv, D, _stream(stream)))


def pa_stream_read(buf, sink, grid: int, stream=None) -> None:
    """Measurement probe: one sequential read of the whole of ``buf`` (any
    contiguous device tensor, a multiple of 16 bytes); ``sink`` is an int32
    device tensor of at least grid * 4 elements that receives per-wave xors."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or \
            not buf.is_contiguous():
        raise ValueError("pa_stream_read: buf must be a contiguous device tensor")
    if sink.numel() < 4 * int(grid):
        raise ValueError("pa_stream_read: sink holds fewer than grid * 4 words")
    _check("pa_stream_read", _lib().pa_stream_read(
        buf.data_ptr(), buf.numel() * buf.element_size(),
        _dev(sink, torch.int32, "sink", 1), int(grid), _stream(stream)))


def pa_swap_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache,
                   src_ids, dst_ids, stream=None) -> None:
    """Block src_ids[k] of the source pool to block dst_ids[k] of the
    destination pool (either pool on the device or in pinned host memory)."""
    torch = _torch()
    snb, B, Hkv, D = src_key_cache.shape
    dnb = dst_key_cache.shape[0]
    if tuple(dst_key_cache.shape[1:]) != (B, Hkv, D) or \
            src_value_cache.shape != src_key_cache.shape or \
            dst_value_cache.shape != dst_key_cache.shape:
        raise ValueError("pa_swap_blocks: pool block shapes differ")
    if src_ids.shape != dst_ids.shape:
        raise ValueError("pa_swap_blocks: src_ids/dst_ids shapes differ")
    _check("pa_swap_blocks", _lib().pa_swap_blocks(
        _mapped(src_key_cache, torch.float16, "src_key_cache", 4),
        _mapped(src_value_cache, torch.float16, "src_value_cache", 4), snb,
        _mapped(dst_key_cache, torch.float16, "dst_key_cache", 4),
        _mapped(dst_value_cache, torch.float16, "dst_value_cache", 4), dnb,
        _dev(src_ids, torch.int32, "src_ids", 1), _dev(dst_ids, torch.int32, "dst_ids", 1),
        src_ids.numel(), B, Hkv, D, _stream(stream)))


def _decode_common(query, key_cache, value_cache, block_tables, context_lens):
    torch = _torch()
    S, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D):
        raise ValueError("decode: inconsistent head_size / cache shapes")
    if block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("decode: block_tables / context_lens do not match query")
    ptrs = (_dev(query, torch.float16, "query", 3),
            _dev(key_cache, torch.float16, "key_cache", 4),
            _dev(value_cache, torch.float16, "value_cache", 4),
            _dev(block_tables, torch.int32, "block_tables", 2),
            _dev(context_lens, torch.int32, "context_lens", 1))
    return ptrs, (S, H, Hkv, D, B, nb, block_tables.shape[1])


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens,
              scale: float, stream=None) -> None:
    torch = _torch()
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("pa_decode: out shape")
    _check("pa_decode", _lib().pa_decode(
        _dev(out, torch.float16, "out", 3), q, kc, vc, bt, M, cl, S, H, Hkv, D,
        B, nb, float(scale), _stream(stream)))


def pa_decode_splitk(query, key_cache, value_cache, block_tables, context_lens,
                     scale: float, partition_size: int, workspace,
                     stream=None) -> None:
    """workspace: any contiguous device tensor of at least
    pa_splitk_workspace_size(...) bytes (e.g. torch.uint8)."""
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_splitk", _lib().pa_decode_splitk(
        q, kc, vc, bt, M, cl, S, H, Hkv, D, B, nb, float(scale),
        int(partition_size), ws, nbytes, _stream(stream)))


def pa_multi_workspace_size(num_q_tokens: int, num_heads: int, head_size: int,
                            max_blocks_per_seq: int, block_size: int,
                            partition_size: int) -> int:
    return int(_lib().pa_multi_workspace_size(num_q_tokens, num_heads, head_size,
                                           max_blocks_per_seq, block_size,
                                           partition_size))


def pa_decode_multi(out, query, key_cache, value_cache, block_tables, cu_seqlens_q,
                    context_lens, max_q_per_seq: int, scale: float,
                    partition_size: int, workspace, stream=None) -> None:
    """Several query tokens per sequence (rows cu_seqlens_q[i] ..
    cu_seqlens_q[i+1]-1 are the last tokens of sequence i), causal within
    the chunk.  query/out fp16 [num_q_tokens, H, D]."""
    torch = _torch()
    Q, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    S = context_lens.shape[0]
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D) or \
            tuple(out.shape) != (Q, H, D):
        raise ValueError("pa_decode_multi: inconsistent shapes")
    if block_tables.shape[0] != S or cu_seqlens_q.shape != (S + 1,):
        raise ValueError("pa_decode_multi: block_tables / cu_seqlens_q do not match")
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_multi", _lib().pa_decode_multi(
        _dev(out, torch.float16, "out", 3), _dev(query, torch.float16, "query", 3),
        _dev(key_cache, torch.float16, "key_cache", 4),
        _dev(value_cache, torch.float16, "value_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1), Q, int(max_q_per_seq),
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, Hkv, D, B, nb,
        float(scale), int(partition_size), ws, nbytes, _stream(stream)))


def pa_prefill(out, query, key_cache, value_cache, block_tables, cu_seqlens_q,
               context_lens, max_q_per_seq: int, scale: float, stream=None) -> None:
    """pa_decode_multi's rows (causal within each sequence's chunk) for long
    chunks: 128 rows x heads per pass over the keys, no workspace."""
    torch = _torch()
    Q, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    S = context_lens.shape[0]
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D) or \
            tuple(out.shape) != (Q, H, D):
        raise ValueError("pa_prefill: inconsistent shapes")
    if block_tables.shape[0] != S or cu_seqlens_q.shape != (S + 1,):
        raise ValueError("pa_prefill: block_tables / cu_seqlens_q do not match")
    _check("pa_prefill", _lib().pa_prefill(
        _dev(out, torch.float16, "out", 3), _dev(query, torch.float16, "query", 3),
        _dev(key_cache, torch.float16, "key_cache", 4),
        _dev(value_cache, torch.float16, "value_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1), Q, int(max_q_per_seq),
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, Hkv, D, B, nb,
        float(scale), _stream(stream)))


def pa_decode_multi_balanced(out, query, key_cache, value_cache, block_tables,
                             cu_seqlens_q, context_lens, max_q_per_seq: int, scale: float,
                             grid: int, workspace, stream=None) -> None:
    """pa_decode_multi on the balanced split, one kernel (T*g <= 16 per
    sequence); workspace zero-filled before its first use."""
    torch = _torch()
    Q, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    S = context_lens.shape[0]
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D) or tuple(out.shape) != (Q, H, D):
        raise ValueError("pa_decode_multi_balanced: inconsistent shapes")
    if block_tables.shape[0] != S or tuple(cu_seqlens_q.shape) != (S + 1,):
        raise ValueError("pa_decode_multi_balanced: block_tables / cu_seqlens_q do not match")
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_multi_balanced", _lib().pa_decode_multi_balanced(
        _dev(out, torch.float16, "out", 3), _dev(query, torch.float16, "query", 3),
        _dev(key_cache, torch.float16, "key_cache", 4),
        _dev(value_cache, torch.float16, "value_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1), Q, int(max_q_per_seq),
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, Hkv, D, B, nb,
        float(scale), int(grid), ws, nbytes, _stream(stream)))


def pa_decode_reduce(out, workspace, context_lens, max_blocks_per_seq: int,
                     block_size: int, partition_size: int, stream=None) -> None:
    torch = _torch()
    S, H, D = out.shape
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_reduce", _lib().pa_decode_reduce(
        _dev(out, torch.float16, "out", 3), ws, nbytes,
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, D,
        int(max_blocks_per_seq), int(block_size), int(partition_size),
        _stream(stream)))


def pa_decode_balanced(out, query, key_cache, value_cache, block_tables,
                       context_lens, scale: float, grid: int, workspace,
                       stream=None) -> None:
    """Balanced split-KV decode (one kernel); workspace: a contiguous device
    tensor of at least pa_balanced_workspace_size(...) bytes, zero-filled
    before its first use (each call leaves its counters at zero)."""
    torch = _torch()
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("pa_decode_balanced: out shape")
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_balanced", _lib().pa_decode_balanced(
        _dev(out, torch.float16, "out", 3), q, kc, vc, bt, M, cl, S, H, Hkv, D, B, nb,
        float(scale), int(grid), ws, nbytes, _stream(stream)))


def pa_decode_balanced_fp8(out, query, key_cache, value_cache, block_tables,
                           context_lens, scale: float, k_scale: float, v_scale: float,
                           grid: int, workspace, stream=None) -> None:
    """Balanced split-KV decode over an fp8 pool (uint8 or float8_e4m3fn
    [nb, B, H_kv, D] halves; stored value = code * k_scale / v_scale)."""
    torch = _torch()
    S, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D):
        raise ValueError("decode: inconsistent head_size / cache shapes")
    if block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("decode: block_tables / context_lens do not match query")
    if tuple(out.shape) != (S, H, D):
        raise ValueError("pa_decode_balanced_fp8: out shape")
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_balanced_fp8", _lib().pa_decode_balanced_fp8(
        _dev(out, torch.float16, "out", 3), _dev(query, torch.float16, "query", 3),
        _dev_fp8(key_cache, "key_cache", 4), _dev_fp8(value_cache, "value_cache", 4),
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, Hkv, D, B, nb,
        float(scale), float(k_scale), float(v_scale), int(grid), ws, nbytes,
        _stream(stream)))


def pa_decode_shared_prefix(out, query, key_cache, value_cache, block_tables,
                            context_lens, scale: float, partition_size: int,
                            group_offsets, group_members, group_blocks,
                            max_group_size: int, max_group_blocks: int, workspace,
                            stream=None) -> None:
    """Split-K decode where each group's shared full blocks are read once for
    all its members (group_* int32 device tensors: CSR member lists and the
    shared leading block count per group)."""
    torch = _torch()
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("pa_decode_shared_prefix: out shape")
    G = int(group_blocks.numel())
    if tuple(group_offsets.shape) != (G + 1,):
        raise ValueError("pa_decode_shared_prefix: group_offsets must have num_groups + 1 entries")
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_shared_prefix", _lib().pa_decode_shared_prefix(
        _dev(out, torch.float16, "out", 3), q, kc, vc, bt, M, cl, S, H, Hkv, D, B, nb,
        float(scale), int(partition_size),
        _dev(group_offsets, torch.int32, "group_offsets", 1),
        _dev(group_members, torch.int32, "group_members", 1),
        _dev(group_blocks, torch.int32, "group_blocks", 1), G, int(max_group_size),
        int(max_group_blocks), ws, nbytes, _stream(stream)))


def pa_decode_step_fp8(out, query, key, value, key_cache, value_cache, block_tables,
                       context_lens, scale: float, k_scale: float, v_scale: float,
                       grid: int, workspace, slot_mapping=None, stream=None) -> None:
    """pa_decode_step over an fp8 pool: key/value ([S, H_kv, D] fp16) are
    quantised into their slots and attended to in that form."""
    torch = _torch()
    S, H, D = query.shape
    nb, B, Hkv, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != (nb, B, Hkv, D):
        raise ValueError("decode: inconsistent head_size / cache shapes")
    if block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("decode: block_tables / context_lens do not match query")
    if tuple(out.shape) != (S, H, D) or tuple(key.shape) != (S, Hkv, D) \
            or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("pa_decode_step_fp8: shapes")
    sm = None if slot_mapping is None else _dev(slot_mapping, torch.int32,
                                                "slot_mapping", 1)
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_step_fp8", _lib().pa_decode_step_fp8(
        _dev(out, torch.float16, "out", 3), _dev(query, torch.float16, "query", 3),
        _dev(key, torch.float16, "key", 3), _dev(value, torch.float16, "value", 3),
        _dev_fp8(key_cache, "key_cache", 4), _dev_fp8(value_cache, "value_cache", 4), sm,
        _dev(block_tables, torch.int32, "block_tables", 2), block_tables.shape[1],
        _dev(context_lens, torch.int32, "context_lens", 1), S, H, Hkv, D, B, nb,
        float(scale), float(k_scale), float(v_scale), int(grid), ws, nbytes,
        _stream(stream)))


def pa_decode_step(out, query, key, value, key_cache, value_cache, block_tables,
                   context_lens, scale: float, grid: int, workspace,
                   slot_mapping=None, stream=None) -> None:
    """One fused decode step: append key/value ([S, H_kv, D] fp16) at position
    context_lens-1 of every sequence, then attend over context_lens tokens.
    slot_mapping (int32 [S], optional) receives the slots written."""
    torch = _torch()
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    if tuple(out.shape) != (S, H, D) or tuple(key.shape) != (S, Hkv, D) \
            or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("pa_decode_step: shapes")
    sm = None if slot_mapping is None else _dev(slot_mapping, torch.int32,
                                                "slot_mapping", 1)
    ws = _dev(workspace, workspace.dtype, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("pa_decode_step", _lib().pa_decode_step(
        _dev(out, torch.float16, "out", 3), q, _dev(key, torch.float16, "key", 3),
        _dev(value, torch.float16, "value", 3), kc, vc, sm, bt, M, cl, S, H, Hkv, D,
        B, nb, float(scale), int(grid), ws, nbytes, _stream(stream)))



def pa_decode_step_noalloc(out, query, key, value, key_cache, value_cache, block_tables,
                           context_lens, scale: float, grid: int, slot_mapping=None,
                           stream=None) -> None:
    """pa_decode_step without a workspace: the library's static device
    array holds the range counters and partial states (no allocation)."""
    torch = _torch()
    (q, kc, vc, bt, cl), (S, H, Hkv, D, B, nb, M) = _decode_common(
        query, key_cache, value_cache, block_tables, context_lens)
    if tuple(out.shape) != (S, H, D) or tuple(key.shape) != (S, Hkv, D) \
            or tuple(value.shape) != (S, Hkv, D):
        raise ValueError("pa_decode_step_noalloc: shapes")
    sm = None if slot_mapping is None else _dev(slot_mapping, torch.int32,
                                                "slot_mapping", 1)
    _check("pa_decode_step_noalloc", _lib().pa_decode_step_noalloc(
        _dev(out, torch.float16, "out", 3), q, _dev(key, torch.float16, "key", 3),
        _dev(value, torch.float16, "value", 3), kc, vc, sm, bt, M, cl, S, H, Hkv, D,
        B, nb, float(scale), int(grid), _stream(stream)))
