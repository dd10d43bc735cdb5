"""Python binding for libpagedkv.so: block-paged KV attention on MI355X.

Argument marshalling only. Every step of the hot path runs in the library's
HIP kernels; PyTorch supplies device memory (tensors) and the current stream.
The module raises ImportError at import time when the library is not built:
there is no fallback path.

The functions mirror the C ABI in ``include/pagedkv.h`` (same names); tensor
arguments are checked for shape, dtype, device and contiguity here, because
the C layer sees only raw pointers.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PAGED_OK = 0
PAGED_ERR_INVALID_ARG = -1
PAGED_ERR_DTYPE = -2
PAGED_ERR_NO_BLOCKS = -3
PAGED_ERR_CAPACITY = -4
PAGED_ERR_STATE = -5
PAGED_ERR_HIP = -6

PAGED_F32 = 0
PAGED_BF16 = 1
PAGED_FP8_E4M3 = 2

KERNELS = {
    "kv_write": 0,
    "kv_gather": 1,
    "decode_partial": 2,
    "decode_reduce": 3,
    "prefill": 4,
    "prefill_reduce": 5,
}

_c_int32 = ctypes.c_int32
_c_int64 = ctypes.c_int64
_c_size = ctypes.c_size_t
_c_void_p = ctypes.c_void_p
_c_float = ctypes.c_float
_c_uint64 = ctypes.c_uint64
_P_I32 = ctypes.POINTER(ctypes.c_int32)
_P_I64 = ctypes.POINTER(ctypes.c_int64)


class PagedError(RuntimeError):
    """A libpagedkv call returned a non-zero status (``.code``)."""

    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


# name -> argument types; every function returns int32 unless listed otherwise
_SIGNATURES = {
    "paged_abi_version": [],
    "paged_last_error": [],
    "paged_kv_write": [_c_void_p] * 5 + [_c_int32] * 6 + [_c_void_p],
    "paged_kv_gather": [_c_void_p] * 5 + [_c_int32, _c_void_p, _c_void_p] + [_c_int32] * 8 + [_c_void_p],
    "paged_kv_write_fp8": [_c_void_p] * 5 + [_c_int32] * 6 + [_c_float] * 2 + [_c_void_p],
    "paged_attn_decode_fp8": [_c_void_p] * 5 + [_c_int32, _c_void_p] + [_c_int32] * 6 + [_c_float] * 3
    + [_c_int32] * 3 + [_c_void_p, _c_size, _c_void_p],
    "paged_attn_prefill_chunk_fp8": [_c_void_p] * 5 + [_c_int32, _c_void_p, _c_void_p] + [_c_int32] * 8
    + [_c_float] * 3 + [_c_int32, _c_void_p, _c_size, _c_void_p],
    "paged_attn_prefill_chunk_workspace_bytes": [_c_int32] * 6 + [ctypes.POINTER(_c_size)],
    "paged_attn_mixed": [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int32, _c_void_p,
                         _c_void_p, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32, _c_int32,
                         _c_int32, _c_int32, _c_int32, _c_float, _c_float, _c_float, _c_int32,
                         _c_int32, _c_int32, _c_void_p, _c_size, _c_int32, _c_void_p],
    "paged_attn_decode_partition_tokens": [_c_int32] * 8 + [_P_I32],
    "paged_attn_decode_workspace_bytes": [_c_int32] * 9 + [ctypes.POINTER(_c_size)],
    "paged_attn_decode": [_c_void_p] * 5 + [_c_int32, _c_void_p] + [_c_int32] * 6 + [_c_float]
    + [_c_int32] * 3 + [_c_void_p, _c_size, _c_int32, _c_void_p],
    "paged_attn_decode_noalloc": [_c_void_p] * 5 + [_c_int32, _c_void_p] + [_c_int32] * 6 + [_c_float]
    + [_c_int32] * 4 + [_c_void_p],
    "paged_attn_prefill_chunk": [_c_void_p] * 5 + [_c_int32, _c_void_p, _c_void_p] + [_c_int32] * 8
    + [_c_float, _c_int32, _c_void_p, _c_size, _c_int32, _c_void_p],
    "paged_trace_enable": [_c_int32],
    "paged_trace_reset": [],
    "paged_trace_query": [_c_int32, ctypes.POINTER(ctypes.c_double), _P_I64],
    "paged_trace_durations": [_c_int32, ctypes.POINTER(ctypes.c_double), _c_int64, _P_I64],
    "paged_alloc_create": [_c_int32, _c_int32, _P_I32, ctypes.POINTER(_c_void_p)],
    "paged_alloc_destroy": [_c_void_p],
    "paged_alloc_grow": [_c_void_p, _c_int32, _P_I32],
    "paged_alloc_num_blocks": [_c_void_p, _P_I32],
    "paged_alloc_set_max_blocks": [_c_void_p, _c_int32],
    "paged_alloc_num_free": [_c_void_p, _P_I32, _P_I32],
    "paged_seq_add": [_c_void_p, _c_int64],
    "paged_seq_match_prefix": [_c_void_p, _c_int64, _P_I32, _c_int32, _c_uint64, _P_I32],
    "paged_seq_share_prefix": [_c_void_p, _c_int64, _c_int64, _c_int32],
    "paged_seq_reserve": [_c_void_p, _c_int64, _c_int32],
    "paged_seq_reserve_or_grow": [_c_void_p, _c_int64, _c_int32, _P_I32],
    "paged_seq_commit_tokens": [_c_void_p, _c_int64, _P_I32, _c_int32],
    "paged_seq_publish_full_blocks": [_c_void_p, _c_int64, _c_uint64],
    "paged_seq_drop_outside_window": [_c_void_p, _c_int64, _c_int32],
    "paged_seq_release": [_c_void_p, _c_int64],
    "paged_seq_num_tokens": [_c_void_p, _c_int64, _P_I32, _P_I32],
    "paged_alloc_block_tables": [_c_void_p, _P_I64, _c_int32, _c_int32, _P_I32, _P_I32],
    "paged_alloc_slot_mapping": [_c_void_p, _c_int64, _c_int32, _c_int32, _P_I64],
    "paged_alloc_refcount": [_c_void_p, _c_int32, _P_I32],
}


def _load():
    # torch wheels ship their own HIP runtime under the same soname as the
    # system one. Importing torch first makes the library bind to that
    # already-loaded runtime, so the process holds exactly one HIP runtime
    # (loading the library first would let torch bring in a second one).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python block_paged_kv_amd/build.py` "
            "(the HIP library is required: there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "paged_last_error" else _c_int32
    return lib


lib = _load()


def _check(rc):
    if rc != PAGED_OK:
        raise PagedError(rc, lib.paged_last_error().decode(errors="replace"))


def _invoke(fn, args, prepare):
    """Call now, or (prepare=True) return a zero-argument callable that repeats
    the call with the same, already converted arguments (for hot loops)."""
    if prepare:
        def call():
            _check(fn(*args))
        return call
    _check(fn(*args))
    return None


def abi_version():
    return lib.paged_abi_version()


# ------------------------------------------------------------------ tensors
def _torch():
    import torch  # imported lazily: the allocator needs no torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PAGED_BF16
    if t.dtype == torch.float32:
        return PAGED_F32
    if t.dtype == torch.float8_e4m3fn:
        return PAGED_FP8_E4M3
    raise PagedError(PAGED_ERR_DTYPE, f"unsupported tensor dtype {t.dtype}")


def _dev(t, name, dtype=None, ndim=None):
    if not t.is_cuda:
        raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PagedError(PAGED_ERR_DTYPE, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _pool_geom(k_pool, v_pool):
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype or k_pool.dim() != 4:
        raise PagedError(PAGED_ERR_INVALID_ARG,
                         "k_pool/v_pool must be equal [num_blocks, num_kv_heads, block_size, head_dim] tensors")
    return tuple(int(x) for x in k_pool.shape)


def paged_kv_write(k_pool, v_pool, new_k, new_v, slot_mapping, stream=None, prepare=False):
    """Scatter ``new_k/new_v [T, Hkv, D]`` into the pools at ``slot_mapping [T]`` (int64)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    T = int(slot_mapping.shape[0])
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        if tuple(t.shape) != (T, hkv, d) or t.dtype != k_pool.dtype:
            raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must be [{T}, {hkv}, {d}] {k_pool.dtype}")
    return _invoke(lib.paged_kv_write, (
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(new_k, "new_k"), _dev(new_v, "new_v"),
        _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, nb, bs, hkv, d,
        _dtype_code(k_pool), _stream(stream)), prepare)


def paged_kv_gather(out_k, out_v, k_pool, v_pool, block_tables, seq_lens, out_offsets,
                    max_seq_len, sliding_window=0, stream=None, prepare=False):
    """Copy each row's attended positions into ``out_k/out_v [sum spans, Hkv, D]``."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    B, mb = (int(x) for x in block_tables.shape)
    if tuple(seq_lens.shape) != (B,) or tuple(out_offsets.shape) != (B,):
        raise PagedError(PAGED_ERR_INVALID_ARG, "seq_lens and out_offsets must be [batch]")
    for name, t in (("out_k", out_k), ("out_v", out_v)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (hkv, d) or t.dtype != k_pool.dtype:
            raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must be [N, {hkv}, {d}] {k_pool.dtype}")
    return _invoke(lib.paged_kv_gather, (
        _dev(out_k, "out_k"), _dev(out_v, "out_v"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32, 2), mb, _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(out_offsets, "out_offsets", torch.int64, 1), B, int(max_seq_len), hkv, d, bs, nb,
        int(sliding_window), _dtype_code(k_pool), _stream(stream)), prepare)


def _dtype_arg(dtype):
    """PAGED_F32 / PAGED_BF16 from a torch dtype, a name or the code itself."""
    if isinstance(dtype, int):
        return dtype
    name = str(dtype).replace("torch.", "")
    codes = {"float32": PAGED_F32, "f32": PAGED_F32, "bfloat16": PAGED_BF16, "bf16": PAGED_BF16,
             "float8_e4m3fn": PAGED_FP8_E4M3, "fp8": PAGED_FP8_E4M3}
    if name not in codes:
        raise PagedError(PAGED_ERR_DTYPE, f"unsupported dtype {dtype}")
    return codes[name]


def paged_attn_decode_partition_tokens(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_seq_len, sliding_window=0, dtype="bf16"):
    out = ctypes.c_int32()
    _check(lib.paged_attn_decode_partition_tokens(batch, num_q_heads, num_kv_heads, head_dim,
                                                  block_size, max_seq_len, sliding_window,
                                                  _dtype_arg(dtype), ctypes.byref(out)))
    return out.value


def paged_attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_seq_len, sliding_window=0, partition_tokens=0,
                                      dtype="bf16"):
    out = _c_size()
    _check(lib.paged_attn_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_seq_len, sliding_window,
                                                 partition_tokens, _dtype_arg(dtype),
                                                 ctypes.byref(out)))
    return out.value


def paged_attn_decode(out, q, k_pool, v_pool, block_tables, seq_lens, scale, max_seq_len,
                      sliding_window=0, partition_tokens=0, workspace=None, stream=None,
                      prepare=False):
    """GQA decode: ``out, q [B, Hq, D]``; tables ``[B, MB]`` int32; ``seq_lens [B]`` int32.

    ``workspace`` is a uint8 device tensor of at least
    ``paged_attn_decode_workspace_bytes(...)`` bytes (None when that is 0).
    """
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    B, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (B, hq, d) or q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [B, Hq, D] in the pool dtype")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != B or tuple(seq_lens.shape) != (B,):
        raise PagedError(PAGED_ERR_INVALID_ARG, "block_tables must be [B, MB] and seq_lens [B]")
    mb = int(block_tables.shape[1])
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    return _invoke(lib.paged_attn_decode, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), mb, _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, hq, hkv, d, bs, nb, float(scale), int(sliding_window), int(partition_tokens),
        int(max_seq_len), ws_ptr, ws_bytes, _dtype_code(q), _stream(stream)), prepare)


def paged_attn_decode_noalloc(out, q, k_pool, v_pool, block_tables, seq_lens, scale, max_seq_len,
                              sliding_window=0, partition_tokens=0, stream=None, prepare=False):
    """``paged_attn_decode`` with the partials in the library's per-GPU device
    scratch (no workspace argument; calls that overlap on one GPU race)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    B, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (B, hq, d) or q.dtype != k_pool.dtype or out.dtype != q.dtype:
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [B, Hq, D] in the pool dtype")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != B or tuple(seq_lens.shape) != (B,):
        raise PagedError(PAGED_ERR_INVALID_ARG, "block_tables must be [B, MB] and seq_lens [B]")
    return _invoke(lib.paged_attn_decode_noalloc, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(seq_lens, "seq_lens", torch.int32, 1), B, hq, hkv, d, bs, nb, float(scale),
        int(sliding_window), int(partition_tokens), int(max_seq_len), _dtype_code(q), _stream(stream)),
        prepare)


def paged_attn_prefill_chunk_workspace_bytes(batch, total_q, max_q_len, num_q_heads, num_kv_heads,
                                             head_dim):
    """Workspace bytes of the prefill's key split for these shapes (0: none)."""
    out = _c_size()
    _check(lib.paged_attn_prefill_chunk_workspace_bytes(batch, total_q, max_q_len, num_q_heads,
                                                        num_kv_heads, head_dim, ctypes.byref(out)))
    return out.value


def _workspace(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()


def paged_attn_prefill_chunk(out, q, k_pool, v_pool, block_tables, cu_q_lens, seq_lens, max_q_len,
                             scale, sliding_window=0, workspace=None, stream=None, prepare=False):
    """Chunked prefill: ``out, q [T, Hq, D]`` bf16; ``cu_q_lens [B+1]``, ``seq_lens [B]`` int32.

    ``workspace``: None (no key split), or a uint8 device tensor of at least
    ``paged_attn_prefill_chunk_workspace_bytes(...)`` bytes."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    T, hq, dq = (int(x) for x in q.shape)
    B = int(seq_lens.shape[0])
    if dq != d or tuple(out.shape) != (T, hq, d) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [T, Hq, D] in the pool dtype")
    if tuple(cu_q_lens.shape) != (B + 1,) or block_tables.dim() != 2 or int(block_tables.shape[0]) != B:
        raise PagedError(PAGED_ERR_INVALID_ARG, "cu_q_lens must be [B+1] and block_tables [B, MB]")
    return _invoke(lib.paged_attn_prefill_chunk, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(cu_q_lens, "cu_q_lens", torch.int32, 1), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, T, int(max_q_len), hq, hkv, d, bs, nb, float(scale), int(sliding_window),
        *_workspace(workspace), _dtype_code(q), _stream(stream)), prepare)


def paged_attn_mixed(out, q, k_pool, v_pool, block_tables, cu_q_lens, seq_lens, num_decode_rows,
                     max_q_len, scale, max_seq_len, sliding_window=0, partition_tokens=0,
                     workspace=None, k_scale=1.0, v_scale=1.0, stream=None, prepare=False):
    """One continuous-batching step: rows ``[0, num_decode_rows)`` are decode rows
    (one query each), the rest prefill chunks; ``out, q [T, Hq, D]`` bf16, pools bf16
    or float8_e4m3fn (then ``k_scale``/``v_scale``). ``workspace`` as for
    ``paged_attn_decode`` over the decode rows."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geom(k_pool, v_pool)
    T, hq, dq = (int(x) for x in q.shape)
    B = int(seq_lens.shape[0])
    if q.dtype != torch.bfloat16 or out.dtype != q.dtype or dq != d or tuple(out.shape) != (T, hq, d):
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [T, Hq, D] bf16")
    if tuple(cu_q_lens.shape) != (B + 1,) or block_tables.dim() != 2 or int(block_tables.shape[0]) != B:
        raise PagedError(PAGED_ERR_INVALID_ARG, "cu_q_lens must be [B+1] and block_tables [B, MB]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    return _invoke(lib.paged_attn_mixed, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(cu_q_lens, "cu_q_lens", torch.int32, 1), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, int(num_decode_rows), T, int(max_q_len), hq, hkv, d, bs, nb, float(scale), float(k_scale),
        float(v_scale), int(sliding_window), int(partition_tokens), int(max_seq_len), ws_ptr, ws_bytes,
        _dtype_code(k_pool), _stream(stream)), prepare)


# ------------------------------------------------------------------ FP8 KV pools
def _fp8_pools(k_pool, v_pool):
    torch = _torch()
    geom = _pool_geom(k_pool, v_pool)
    if k_pool.dtype != torch.float8_e4m3fn:
        raise PagedError(PAGED_ERR_DTYPE, f"FP8 pools must be torch.float8_e4m3fn, got {k_pool.dtype}")
    return geom


def paged_kv_write_fp8(k_pool, v_pool, new_k, new_v, slot_mapping, k_scale, v_scale, stream=None,
                       prepare=False):
    """Quantizing write: ``new_k/new_v [T, Hkv, D]`` (bf16 or f32) into float8_e4m3fn pools."""
    torch = _torch()
    nb, hkv, bs, d = _fp8_pools(k_pool, v_pool)
    T = int(slot_mapping.shape[0])
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        if tuple(t.shape) != (T, hkv, d) or t.dtype != new_k.dtype:
            raise PagedError(PAGED_ERR_INVALID_ARG, f"{name} must be [{T}, {hkv}, {d}] like new_k")
    return _invoke(lib.paged_kv_write_fp8, (
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(new_k, "new_k"), _dev(new_v, "new_v"),
        _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, nb, bs, hkv, d,
        _dtype_code(new_k), float(k_scale), float(v_scale), _stream(stream)), prepare)


def paged_attn_decode_fp8(out, q, k_pool, v_pool, block_tables, seq_lens, scale, k_scale, v_scale,
                          max_seq_len, sliding_window=0, partition_tokens=0, workspace=None,
                          stream=None, prepare=False):
    """GQA decode over float8_e4m3fn pools; ``out, q [B, Hq, D]`` bf16."""
    torch = _torch()
    nb, hkv, bs, d = _fp8_pools(k_pool, v_pool)
    B, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (B, hq, d) or q.dtype != torch.bfloat16 or out.dtype != q.dtype:
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [B, Hq, D] bf16")
    if block_tables.dim() != 2 or int(block_tables.shape[0]) != B or tuple(seq_lens.shape) != (B,):
        raise PagedError(PAGED_ERR_INVALID_ARG, "block_tables must be [B, MB] and seq_lens [B]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    return _invoke(lib.paged_attn_decode_fp8, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(seq_lens, "seq_lens", torch.int32, 1), B, hq, hkv, d, bs, nb, float(scale),
        float(k_scale), float(v_scale), int(sliding_window), int(partition_tokens), int(max_seq_len),
        ws_ptr, ws_bytes, _stream(stream)), prepare)


def paged_attn_prefill_chunk_fp8(out, q, k_pool, v_pool, block_tables, cu_q_lens, seq_lens,
                                 max_q_len, scale, k_scale, v_scale, sliding_window=0, workspace=None,
                                 stream=None, prepare=False):
    """Chunked prefill over float8_e4m3fn pools; ``out, q [T, Hq, D]`` bf16."""
    torch = _torch()
    nb, hkv, bs, d = _fp8_pools(k_pool, v_pool)
    T, hq, dq = (int(x) for x in q.shape)
    B = int(seq_lens.shape[0])
    if dq != d or tuple(out.shape) != (T, hq, d) or q.dtype != torch.bfloat16 or out.dtype != q.dtype:
        raise PagedError(PAGED_ERR_INVALID_ARG, "q/out must be [T, Hq, D] bf16")
    if tuple(cu_q_lens.shape) != (B + 1,) or block_tables.dim() != 2 or int(block_tables.shape[0]) != B:
        raise PagedError(PAGED_ERR_INVALID_ARG, "cu_q_lens must be [B+1] and block_tables [B, MB]")
    return _invoke(lib.paged_attn_prefill_chunk_fp8, (
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(cu_q_lens, "cu_q_lens", torch.int32, 1), _dev(seq_lens, "seq_lens", torch.int32, 1),
        B, T, int(max_q_len), hq, hkv, d, bs, nb, float(scale), float(k_scale), float(v_scale),
        int(sliding_window), *_workspace(workspace), _stream(stream)), prepare)


# ------------------------------------------------------------------ tracing
def trace_enable(on=True):
    _check(lib.paged_trace_enable(1 if on else 0))


def trace_reset():
    _check(lib.paged_trace_reset())


def trace_query(kernel):
    """(total milliseconds, launches) recorded for ``kernel`` (a KERNELS name)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib.paged_trace_query(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def trace_durations(kernel):
    """Per-launch durations (ms, numpy float64) recorded for ``kernel``, in launch order."""
    n = ctypes.c_int64()
    _check(lib.paged_trace_durations(KERNELS[kernel], None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=np.float64)
    if n.value:
        _check(lib.paged_trace_durations(KERNELS[kernel], out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                         n.value, ctypes.byref(n)))
    return out


# ------------------------------------------------------------------ allocator
def _i32_array(values):
    arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return arr, arr.ctypes.data_as(_P_I32)


class Allocator:
    """Host block allocator (``paged_alloc_*`` / ``paged_seq_*``) for one pool."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self.bs = int(block_size)
        handle = _c_void_p()
        keep = None
        ptr = None
        if free_order is not None:
            keep, ptr = _i32_array(free_order)
            if keep.shape[0] != num_blocks - 1:
                raise PagedError(PAGED_ERR_INVALID_ARG, "free_order must have num_blocks - 1 entries")
        _check(lib.paged_alloc_create(int(num_blocks), int(block_size), ptr, ctypes.byref(handle)))
        self._h = handle
        del keep

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.paged_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass

    @property
    def nb(self):
        out = ctypes.c_int32()
        _check(lib.paged_alloc_num_blocks(self._h, ctypes.byref(out)))
        return out.value

    def grow(self, new_num_blocks, new_order=None):
        keep, ptr = (None, None) if new_order is None else _i32_array(new_order)
        _check(lib.paged_alloc_grow(self._h, int(new_num_blocks), ptr))

    def set_max_blocks(self, max_blocks):
        _check(lib.paged_alloc_set_max_blocks(self._h, int(max_blocks)))

    def reserve_or_grow(self, seq_id, total_tokens):
        """0 when reserved; else the block count the pools must grow to first
        (grow, then retry with ``reserve``)."""
        out = ctypes.c_int32()
        _check(lib.paged_seq_reserve_or_grow(self._h, int(seq_id), int(total_tokens), ctypes.byref(out)))
        return out.value

    def num_free(self):
        f, e = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.paged_alloc_num_free(self._h, ctypes.byref(f), ctypes.byref(e)))
        return f.value, e.value

    def add(self, seq_id):
        _check(lib.paged_seq_add(self._h, int(seq_id)))

    def match_prefix(self, seq_id, tokens, domain):
        arr, ptr = _i32_array(tokens)
        out = ctypes.c_int32()
        _check(lib.paged_seq_match_prefix(self._h, int(seq_id), ptr, int(arr.shape[0]),
                                          int(domain), ctypes.byref(out)))
        return out.value

    def share_prefix(self, dst_id, src_id, num_blocks):
        _check(lib.paged_seq_share_prefix(self._h, int(dst_id), int(src_id), int(num_blocks)))

    def reserve(self, seq_id, total_tokens):
        _check(lib.paged_seq_reserve(self._h, int(seq_id), int(total_tokens)))

    def commit_tokens(self, seq_id, tokens):
        arr, ptr = _i32_array(tokens)
        _check(lib.paged_seq_commit_tokens(self._h, int(seq_id), ptr, int(arr.shape[0])))

    def publish_full_blocks(self, seq_id, domain):
        _check(lib.paged_seq_publish_full_blocks(self._h, int(seq_id), int(domain)))

    def drop_outside_window(self, seq_id, window):
        _check(lib.paged_seq_drop_outside_window(self._h, int(seq_id), int(window)))

    def release(self, seq_id):
        _check(lib.paged_seq_release(self._h, int(seq_id)))

    def _counts(self, seq_id):
        t, b = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.paged_seq_num_tokens(self._h, int(seq_id), ctypes.byref(t), ctypes.byref(b)))
        return t.value, b.value

    def num_tokens(self, seq_id):
        return self._counts(seq_id)[0]

    def num_blocks_of(self, seq_id):
        return self._counts(seq_id)[1]

    def block_tables(self, seq_ids, max_blocks):
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        out = np.zeros((ids.shape[0], int(max_blocks)), dtype=np.int32)
        needed = ctypes.c_int32()
        _check(lib.paged_alloc_block_tables(self._h, ids.ctypes.data_as(_P_I64), int(ids.shape[0]),
                                            int(max_blocks), out.ctypes.data_as(_P_I32),
                                            ctypes.byref(needed)))
        return out

    def slot_mapping(self, seq_id, start_pos, n):
        out = np.zeros(int(n), dtype=np.int64)
        _check(lib.paged_alloc_slot_mapping(self._h, int(seq_id), int(start_pos), int(n),
                                            out.ctypes.data_as(_P_I64)))
        return out

    def refcount(self, block_id):
        out = ctypes.c_int32()
        _check(lib.paged_alloc_refcount(self._h, int(block_id), ctypes.byref(out)))
        return out.value
