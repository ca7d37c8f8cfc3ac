"""Paged KV-cache decode attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding of libpa.so, the C ABI declared in include/pa.h.  Every
function here only checks and marshals arguments (device pointers, sizes,
torch's current HIP stream) and calls the library; all arithmetic runs in the
HIP kernels.  There is no fallback: if libpa.so is missing or a tensor is not
on the GPU, the call raises.

    cache_write(k, v, k_cache, v_cache, slot_mapping)
    decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, ...)
    reduce(out, workspace, context_lens, ...)
    decode_workspace_size(...), new_workspace(...)
    paged_attention(...)   # decode, plus reduce when the context is split
    cache_write_fp8(...), decode_fp8(...)   # the same over an fp8 (E4M3) cache with per-head scales
    copy_blocks(...)       # whole-block copies (copy-on-write, swapping)
    kv_cache_layout(...), allocate_kv_cache(...)   # one layer's K and V pools in one allocation
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PA_F32", "PA_BF16", "PA_BALANCED", "PagedAttentionError", "library_path", "load_library", "status_string", "version",
    "cache_write", "decode", "reduce", "decode_workspace_size", "paged_attention", "cache_write_fp8", "decode_fp8",
    "decode_tree", "prefill", "copy_blocks", "decode_balanced_noalloc", "decode_append", "kv_cache_layout", "allocate_kv_cache", "SYMBOLS",
]

PA_F32, PA_BF16 = 0, 1
PA_BALANCED = -1  # partition_size selecting the work-balanced decode
BLOCK_SIZE = 16
SYMBOLS = ("pa_cache_write", "pa_decode", "pa_decode_workspace_size", "pa_reduce", "pa_status_string", "pa_version",
           "pa_cache_write_fp8", "pa_decode_fp8", "pa_decode_tree", "pa_prefill", "pa_copy_blocks",
           "pa_decode_balanced_noalloc", "pa_decode_append", "pa_kv_cache_layout")
_STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED", 4: "PA_ERR_WORKSPACE",
           5: "PA_ERR_HIP", 6: "PA_ERR_MEMORY", 7: "PA_ERR_SCRATCH"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def library_path() -> str:
    return os.environ.get("PA_LIBRARY", os.path.join(_HERE, "libpa.so"))


def load_library():
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_attention_decode_amd.build`")
    lib = ctypes.CDLL(path)
    i32, i64, f32, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.pa_cache_write.restype = ctypes.c_int
    lib.pa_cache_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz,
                              ctypes.c_int, vp]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode_workspace_size.argtypes = [i32] * 8
    lib.pa_decode_append.restype = ctypes.c_int
    lib.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                     vp, sz, ctypes.c_int, vp]
    lib.pa_decode_balanced_noalloc.restype = ctypes.c_int
    lib.pa_decode_balanced_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32,
                                               ctypes.c_int, vp]
    lib.pa_reduce.restype = ctypes.c_int
    lib.pa_reduce.argtypes = [vp, vp, sz, vp, i32, i32, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pa_cache_write_fp8.restype = ctypes.c_int
    lib.pa_cache_write_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    lib.pa_decode_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                  vp, sz, ctypes.c_int, vp]
    lib.pa_decode_tree.restype = ctypes.c_int
    lib.pa_decode_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                   vp, sz, ctypes.c_int, vp]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                               ctypes.c_int, vp]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int64, vp]
    lib.pa_kv_cache_layout.restype = ctypes.c_int
    lib.pa_kv_cache_layout.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_version.restype = i32
    lib.pa_version.argtypes = []
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


def version() -> int:
    return int(load_library().pa_version())


# ---------------------------------------------------------------------------
# marshalling helpers


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise PagedAttentionError(status, where)


# ---------------------------------------------------------------------------
# the entry points


def cache_write(k, v, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """pa_cache_write: store token t's K/V rows at flat slot slot_mapping[t] (negative = skip)."""
    torch = _torch()
    pk = _dev(k, "k", ndim=3)
    pv = _dev(v, "v", k.dtype, 3)
    pkc = _dev(k_cache, "k_cache", k.dtype, 4)
    pvc = _dev(v_cache, "v_cache", k.dtype, 4)
    ps = _dev(slot_mapping, "slot_mapping", torch.int64, 1)
    T, n_kv, d = k.shape
    if v.shape != k.shape or k_cache.shape != v_cache.shape or tuple(k_cache.shape[2:]) != (n_kv, d):
        raise ValueError("k/v must be [T, n_kv, d] and the caches [num_blocks, block_size, n_kv, d]")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must hold one slot per token")
    st = load_library().pa_cache_write(pk, pv, pkc, pvc, ps, T, k_cache.shape[0], k_cache.shape[1], n_kv, d,
                                       _dtype_code(k), _stream(stream))
    _check(st, "pa_cache_write")


def decode_workspace_size(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, partition_size,
                          block_size=BLOCK_SIZE) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim,
                                                       max_blocks_per_seq, block_size, partition_size))


def new_workspace(q, k_cache, block_tables, q_len: int, partition_size: int):
    """A workspace for decode(..., partition_size): zero-filled, which a balanced
    call needs before its first use (every balanced call leaves it so)."""
    torch = _torch()
    need = decode_workspace_size(block_tables.shape[0], q_len, q.shape[1], k_cache.shape[2], q.shape[2],
                                 block_tables.shape[1], partition_size, k_cache.shape[1])
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)


def _decode_shapes(q, k_cache, block_tables, context_lens, q_len):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [S*q_len, n_h, d] and the caches [num_blocks, block_size, n_kv, d]")
    S = block_tables.shape[0]
    if q.shape[0] != S * q_len:
        raise ValueError(f"q holds {q.shape[0]} rows; expected num_seqs * q_len = {S * q_len}")
    if context_lens.shape != (S,) or context_lens.dtype != torch.int32 or block_tables.dtype != torch.int32:
        raise ValueError("block_tables must be int32 [S, max_blocks] and context_lens int32 [S]")
    return S


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, q_len: int = 1, partition_size: int = 0,
           out=None, workspace=None, stream=None):
    """pa_decode.

    partition_size 0 (one pass) or PA_BALANCED: writes and returns out.
    partition_size > 0: fills the workspace with per-partition partials for
    reduce() and returns the workspace.  A workspace is allocated (zero-filled)
    when none is given; pass the same one again to avoid the allocation.
    """
    torch = _torch()
    S = _decode_shapes(q, k_cache, block_tables, context_lens, q_len)
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    MB = block_tables.shape[1]
    args_common = (_dev(q, "q", ndim=3), _dev(k_cache, "k_cache", q.dtype, 4), _dev(v_cache, "v_cache", q.dtype, 4),
                   _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1))
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    pws, nws = None, 0
    if partition_size != 0:
        if workspace is None:
            workspace = new_workspace(q, k_cache, block_tables, q_len, partition_size)
        pws, nws = _dev(workspace, "workspace", torch.uint8, 1), workspace.numel()
    pout = None
    if partition_size <= 0:
        if out is None:
            out = torch.empty_like(q)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
        pout = _dev(out, "out", q.dtype, 3)
    st = load_library().pa_decode(pout, *args_common, float(scale), q_len, S, n_h, n_kv, d, NB, bs, MB,
                                  partition_size, pws, nws, _dtype_code(q), _stream(stream))
    _check(st, "pa_decode")
    return out if partition_size <= 0 else workspace


def decode_append(q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, scale: float, q_len: int = 1,
                  partition_size: int = 0, out=None, workspace=None, stream=None):
    """pa_decode_append: store the new tokens' K/V rows at their positions (new token j
    of sequence b at L_b - q_len + j, through the block table) and run pa_decode, in
    one launch.  Returns out, or the workspace for reduce() when partition_size > 0."""
    torch = _torch()
    S = _decode_shapes(q, k_cache, block_tables, context_lens, q_len)
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    MB = block_tables.shape[1]
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if new_k.shape != (S * q_len, n_kv, d) or new_v.shape != new_k.shape:
        raise ValueError(f"new_k and new_v must be [num_seqs * q_len, n_kv, d] = {(S * q_len, n_kv, d)}")
    pws, nws = None, 0
    if partition_size != 0:
        if workspace is None:
            workspace = new_workspace(q, k_cache, block_tables, q_len, partition_size)
        pws, nws = _dev(workspace, "workspace", torch.uint8, 1), workspace.numel()
    pout = None
    if partition_size <= 0:
        if out is None:
            out = torch.empty_like(q)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
        pout = _dev(out, "out", q.dtype, 3)
    st = load_library().pa_decode_append(
        pout, _dev(q, "q", ndim=3), _dev(new_k, "new_k", q.dtype, 3), _dev(new_v, "new_v", q.dtype, 3),
        _dev(k_cache, "k_cache", q.dtype, 4), _dev(v_cache, "v_cache", q.dtype, 4),
        _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1),
        float(scale), q_len, S, n_h, n_kv, d, NB, bs, MB, partition_size, pws, nws, _dtype_code(q), _stream(stream))
    _check(st, "pa_decode_append")
    return out if partition_size <= 0 else workspace


def decode_balanced_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, q_len: int = 1,
                            out=None, stream=None):
    """pa_decode_balanced_noalloc: the balanced decode on the library's fixed scratch
    (the C call allocates nothing; out is allocated here when not given)."""
    torch = _torch()
    S = _decode_shapes(q, k_cache, block_tables, context_lens, q_len)
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    MB = block_tables.shape[1]
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    st = load_library().pa_decode_balanced_noalloc(
        _dev(out, "out", q.dtype, 3), _dev(q, "q", ndim=3), _dev(k_cache, "k_cache", q.dtype, 4),
        _dev(v_cache, "v_cache", q.dtype, 4), _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(context_lens, "context_lens", torch.int32, 1), float(scale), q_len, S, n_h, n_kv, d, NB, bs, MB,
        _dtype_code(q), _stream(stream))
    _check(st, "pa_decode_balanced_noalloc")
    return out


def reduce(out, workspace, context_lens, q_len: int, max_blocks_per_seq: int, partition_size: int, stream=None):
    """pa_reduce: merge the partials of a split decode into out [S*q_len, n_h, d]."""
    torch = _torch()
    S = context_lens.shape[0]
    n_h, d = out.shape[1], out.shape[2]
    st = load_library().pa_reduce(_dev(out, "out", ndim=3), _dev(workspace, "workspace", torch.uint8, 1),
                                  workspace.numel(), _dev(context_lens, "context_lens", torch.int32, 1), S, q_len,
                                  n_h, d, max_blocks_per_seq, BLOCK_SIZE, partition_size, _dtype_code(out),
                                  _stream(stream))
    _check(st, "pa_reduce")
    return out


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, scale: float, q_len: int = 1,
                    partition_size: int = 0, out=None, workspace=None, stream=None):
    """The whole attention step: pa_decode, followed by pa_reduce when partition_size > 0."""
    torch = _torch()
    if partition_size <= 0:
        return decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, partition_size, out, workspace,
                      stream)
    ws = decode(q, k_cache, v_cache, block_tables, context_lens, scale, q_len, partition_size, None, workspace, stream)
    if out is None:
        out = torch.empty_like(q)
    return reduce(out, ws, context_lens, q_len, block_tables.shape[1], partition_size, stream)


# ---------------------------------------------------------------------------
# fp8 (E4M3) KV cache


def _scales(k_scale, v_scale, n_kv):
    torch = _torch()
    pk = _dev(k_scale, "k_scale", torch.float32, 1)
    pv = _dev(v_scale, "v_scale", torch.float32, 1)
    if k_scale.shape[0] != n_kv or v_scale.shape[0] != n_kv:
        raise ValueError(f"k_scale and v_scale must hold one fp32 scale per KV head ({n_kv})")
    return pk, pv


def cache_write_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=None) -> None:
    """pa_cache_write_fp8: quantize token t's K/V rows (fp32 or bf16) into the uint8
    E4M3 caches at flat slot slot_mapping[t] with the per-head scales."""
    torch = _torch()
    pk = _dev(k, "k", ndim=3)
    pv = _dev(v, "v", k.dtype, 3)
    pkc = _dev(k_cache, "k_cache", torch.uint8, 4)
    pvc = _dev(v_cache, "v_cache", torch.uint8, 4)
    ps = _dev(slot_mapping, "slot_mapping", torch.int64, 1)
    T, n_kv, d = k.shape
    if v.shape != k.shape or k_cache.shape != v_cache.shape or tuple(k_cache.shape[2:]) != (n_kv, d):
        raise ValueError("k/v must be [T, n_kv, d] and the caches [num_blocks, block_size, n_kv, d]")
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must hold one slot per token")
    sk, sv = _scales(k_scale, v_scale, n_kv)
    st = load_library().pa_cache_write_fp8(pk, pv, pkc, pvc, ps, sk, sv, T, k_cache.shape[0], k_cache.shape[1],
                                           n_kv, d, _dtype_code(k), _stream(stream))
    _check(st, "pa_cache_write_fp8")


def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale: float, q_len: int = 1,
               partition_size: int = 0, out=None, workspace=None, stream=None):
    """pa_decode_fp8: decode over uint8 E4M3 caches with per-head scales; q/out bf16.
    Same partition_size / workspace / return conventions as decode()."""
    torch = _torch()
    S = _decode_shapes(q, k_cache, block_tables, context_lens, q_len)
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    MB = block_tables.shape[1]
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    args = (_dev(q, "q", torch.bfloat16, 3), _dev(k_cache, "k_cache", torch.uint8, 4),
            _dev(v_cache, "v_cache", torch.uint8, 4), *_scales(k_scale, v_scale, n_kv),
            _dev(block_tables, "block_tables", torch.int32, 2), _dev(context_lens, "context_lens", torch.int32, 1))
    pws, nws = None, 0
    if partition_size != 0:
        if workspace is None:
            workspace = new_workspace(q, k_cache, block_tables, q_len, partition_size)
        pws, nws = _dev(workspace, "workspace", torch.uint8, 1), workspace.numel()
    pout = None
    if partition_size <= 0:
        if out is None:
            out = torch.empty_like(q)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
        pout = _dev(out, "out", q.dtype, 3)
    st = load_library().pa_decode_fp8(pout, *args, float(scale), q_len, S, n_h, n_kv, d, NB, bs, MB, partition_size,
                                      pws, nws, PA_BF16, _stream(stream))
    _check(st, "pa_decode_fp8")
    return out if partition_size <= 0 else workspace


# ---------------------------------------------------------------------------
# tree verify


def decode_tree(q, k_cache, v_cache, block_tables, context_lens, parents, scale: float, partition_size: int = 0,
                out=None, workspace=None, stream=None):
    """pa_decode_tree: T = parents.shape[1] draft-tree nodes per sequence (q is [S*T, n_h, d],
    bf16), parents int32 [S, T] on the GPU (an earlier node, or -1 for a root).  Same
    partition_size / workspace / return conventions as decode(), with q_len = T."""
    torch = _torch()
    pp = _dev(parents, "parents", torch.int32, 2)
    T = parents.shape[1]
    S = _decode_shapes(q, k_cache, block_tables, context_lens, T)
    if parents.shape[0] != S:
        raise ValueError("parents must be [num_seqs, tree_size]")
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    MB = block_tables.shape[1]
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    args = (_dev(q, "q", torch.bfloat16, 3), _dev(k_cache, "k_cache", torch.bfloat16, 4),
            _dev(v_cache, "v_cache", torch.bfloat16, 4), _dev(block_tables, "block_tables", torch.int32, 2),
            _dev(context_lens, "context_lens", torch.int32, 1), pp)
    pws, nws = None, 0
    if partition_size != 0:
        if workspace is None:
            workspace = new_workspace(q, k_cache, block_tables, T, partition_size)
        pws, nws = _dev(workspace, "workspace", torch.uint8, 1), workspace.numel()
    pout = None
    if partition_size <= 0:
        if out is None:
            out = torch.empty_like(q)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
        pout = _dev(out, "out", q.dtype, 3)
    st = load_library().pa_decode_tree(pout, *args, float(scale), T, S, n_h, n_kv, d, NB, bs, MB, partition_size,
                                       pws, nws, PA_BF16, _stream(stream))
    _check(st, "pa_decode_tree")
    return out if partition_size <= 0 else workspace


# ---------------------------------------------------------------------------
# chunked prefill


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float, max_q_len: int,
            out=None, stream=None):
    """pa_prefill: sequence b owns q rows query_start[b] .. query_start[b+1]-1 (int32 [S+1] on the
    GPU), its new tokens at the last positions of its context; bf16.  max_q_len bounds every
    sequence's count (a host-side figure: the binding does not read query_start back)."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [tokens, n_h, d] and the caches [num_blocks, block_size, n_kv, d]")
    S = block_tables.shape[0]
    if query_start.shape != (S + 1,) or context_lens.shape != (S,):
        raise ValueError("query_start must be [num_seqs + 1] and context_lens [num_seqs]")
    n_h, d = q.shape[1], q.shape[2]
    NB, bs, n_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    st = load_library().pa_prefill(_dev(out, "out", torch.bfloat16, 3), _dev(q, "q", torch.bfloat16, 3),
                                   _dev(k_cache, "k_cache", torch.bfloat16, 4),
                                   _dev(v_cache, "v_cache", torch.bfloat16, 4),
                                   _dev(block_tables, "block_tables", torch.int32, 2),
                                   _dev(context_lens, "context_lens", torch.int32, 1),
                                   _dev(query_start, "query_start", torch.int32, 1), float(scale), S, q.shape[0],
                                   int(max_q_len), n_h, n_kv, d, NB, bs, block_tables.shape[1], PA_BF16,
                                   _stream(stream))
    _check(st, "pa_prefill")
    return out


# ---------------------------------------------------------------------------
# block copies


def _pool(t, name):
    """A cache for copy_blocks: on the GPU, or in pinned host memory (swap space)."""
    torch = _torch()
    if isinstance(t, torch.Tensor) and t.device.type == "cpu" and t.is_pinned():
        if not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-dimensional cache")
        return ctypes.c_void_p(t.data_ptr())
    return _dev(t, name, ndim=4)


def copy_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None) -> None:
    """pa_copy_blocks: for each row (s, d) of block_mapping (int64 [pairs, 2] on the GPU),
    copy block s of src_k/src_v to block d of dst_k/dst_v as raw bytes.  The caches are
    [num_blocks, block_size, n_kv, d] of any one element type, on the GPU or in pinned
    host memory (swap out / swap in); src and dst may be the same."""
    torch = _torch()
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape or src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("K/V pairs must match, and source and destination blocks must have the same shape")
    if src_k.dtype != dst_k.dtype or src_v.dtype != src_k.dtype or dst_v.dtype != dst_k.dtype:
        raise TypeError("source and destination caches must have the same element type")
    pm = _dev(block_mapping, "block_mapping", torch.int64, 2)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [pairs, 2]")
    block_bytes = src_k[0].numel() * src_k.element_size()
    st = load_library().pa_copy_blocks(_pool(src_k, "src_k"), _pool(src_v, "src_v"),
                                       _pool(dst_k, "dst_k"), _pool(dst_v, "dst_v"), pm,
                                       block_mapping.shape[0], src_k.shape[0], dst_k.shape[0], block_bytes,
                                       _stream(stream))
    _check(st, "pa_copy_blocks")


def kv_cache_layout(num_blocks: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> tuple:
    """pa_kv_cache_layout: (total_bytes, v_offset) of one allocation holding a layer's K pool
    at byte 0 and its V pool at v_offset, each [num_blocks, 16, num_kv_heads, head_dim] of
    elem_bytes-byte elements.  A host-side query; needs no GPU."""
    total, voff = ctypes.c_int64(0), ctypes.c_int64(0)
    st = load_library().pa_kv_cache_layout(num_blocks, BLOCK_SIZE, num_kv_heads, head_dim, elem_bytes,
                                           ctypes.byref(total), ctypes.byref(voff))
    _check(st, "pa_kv_cache_layout")
    return int(total.value), int(voff.value)


def allocate_kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda") -> tuple:
    """One layer's (k_cache, v_cache), each [num_blocks, 16, num_kv_heads, head_dim] of dtype
    (torch.bfloat16, torch.float32, or torch.uint8 for fp8 codes), placed in one allocation
    as pa_kv_cache_layout says: K at a 2 KiB-aligned base, V one head slice off K's offsets.
    The two tensors are views that keep the allocation alive; contents are uninitialized."""
    torch = _torch()
    elem = torch.empty((), dtype=dtype).element_size()
    total, voff = kv_cache_layout(num_blocks, num_kv_heads, head_dim, elem)
    buf = torch.empty(total + 2048, dtype=torch.uint8, device=device)
    base = (-buf.data_ptr()) % 2048
    pool = num_blocks * BLOCK_SIZE * num_kv_heads * head_dim * elem
    shape = (num_blocks, BLOCK_SIZE, num_kv_heads, head_dim)
    k = buf[base:base + pool].view(dtype).view(shape)
    v = buf[base + voff:base + voff + pool].view(dtype).view(shape)
    return k, v
