"""ctypes binding of libpa (include/pa.h).

Argument marshalling only: torch tensors supply device memory and the stream;
every step of the computation runs in the library's HIP kernels.  There is no
fallback: if libpa.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import re
from typing import Optional, Tuple

import torch

# The in-tree build; PA_LIBRARY names another build of the same sources (the
# sanitizer build of the host code that the CPU tests load).
LIB_PATH = pathlib.Path(os.environ.get("PA_LIBRARY") or
                        pathlib.Path(__file__).resolve().parent / "libpa.so").resolve()
INCLUDE = pathlib.Path(__file__).resolve().parent.parent / "include"

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_FLAG_SHARED_KV = 1
PA_FLAG_VALU_ONLY = 2
PA_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/pa.h
_DTYPES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}

_c_int, _c_void_p, _c_size_t, _c_float = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
_SIGNATURES = {
    "pa_abi_version": (_c_int, []),
    "pa_status_str": (ctypes.c_char_p, [_c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_cache_write": (_c_int, [_c_void_p] * 6 + [_c_int] * 7 + [_c_void_p]),
    "pa_decode": (_c_int, [_c_void_p] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_int, _c_void_p]),
    "pa_decode_splitk_workspace_bytes": (_c_size_t, [_c_int] * 5),
    "pa_decode_splitk": (_c_int, [_c_void_p] * 6 + [_c_int] * 7 +
                         [_c_float, _c_int, _c_int, _c_int, _c_void_p, _c_size_t, _c_int,
                          _c_void_p]),
    "pa_write_decode": (_c_int, [_c_void_p] * 8 + [_c_int] * 7 + [_c_float, _c_int, _c_int,
                                                                _c_void_p]),
    "pa_write_decode_splitk": (_c_int, [_c_void_p] * 8 + [_c_int] * 7 +
                               [_c_float, _c_int, _c_int, _c_int, _c_void_p, _c_size_t, _c_int,
                                _c_void_p]),
    "pa_decode_splitk_noalloc": (_c_int, [_c_void_p] * 6 + [_c_int] * 7 +
                                 [_c_float, _c_int, _c_int, _c_int, _c_int, _c_void_p]),
    "pa_cache_write_contiguous": (_c_int, [_c_void_p] * 5 + [_c_int] * 5 + [_c_void_p]),
    "pa_decode_contiguous": (_c_int, [_c_void_p] * 5 + [_c_int] * 5 +
                             [_c_float, _c_int, _c_int, _c_void_p, _c_size_t, _c_int,
                              _c_void_p]),
    "pa_read_probe": (_c_int, [_c_void_p, _c_size_t, _c_void_p, _c_int, _c_void_p, _c_void_p]),
    "pa_device_memory": (_c_int, [_c_int, ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "pa_check_inputs_host": (_c_int, [_c_void_p, _c_void_p] + [_c_int] * 5 +
                             [ctypes.POINTER(_c_int)]),
    "pa_decode_shared_prefix_workspace_bytes": (_c_size_t, [_c_int] * 6),
    "pa_copy_blocks": (_c_int, [_c_void_p] * 3 + [_c_int] * 6 + [_c_void_p]),
    "pa_swap_blocks": (_c_int, [_c_void_p] * 5 + [_c_int] * 3 + [_c_size_t, _c_int, _c_void_p]),
    # block manager (include/pa_block_manager.h)
    "pa_bm_create": (_c_int, [_c_int] * 3 + [ctypes.POINTER(_c_void_p)]),
    "pa_bm_destroy": (None, [_c_void_p]),
    "pa_bm_can_allocate": (_c_int, [_c_void_p, _c_int]),
    "pa_bm_allocate": (_c_int, [_c_void_p, _c_int, _c_int]),
    "pa_bm_append_slot": (_c_int, [_c_void_p, _c_int] + [ctypes.POINTER(ctypes.c_int32)] * 4),
    "pa_bm_fork": (_c_int, [_c_void_p, _c_int, _c_int]),
    "pa_bm_free": (_c_int, [_c_void_p, _c_int]),
    "pa_bm_swap_out": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, ctypes.POINTER(_c_int)]),
    "pa_bm_swap_in": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, ctypes.POINTER(_c_int)]),
    "pa_bm_num_free_blocks": (_c_int, [_c_void_p, _c_int]),
    "pa_bm_usage_ratio": (ctypes.c_double, [_c_void_p]),
    "pa_bm_seq_info": (_c_int, [_c_void_p, _c_int] + [ctypes.POINTER(_c_int)] * 3),
    "pa_bm_refcount": (_c_int, [_c_void_p, _c_int, _c_int]),
    "pa_bm_fill_batch": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_void_p]),
    "pa_bm_prefix_groups": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p,
                                     ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "pa_decode_shared_prefix": (_c_int, [_c_void_p] * 8 + [_c_int] * 7 +
                                [_c_float] + [_c_int] * 5 + [_c_void_p, _c_size_t, _c_int,
                                                              _c_void_p]),
    "pa_write_decode_shared_prefix": (_c_int, [_c_void_p] * 10 + [_c_int] * 7 +
                                      [_c_float] + [_c_int] * 5 + [_c_void_p, _c_size_t,
                                                                    _c_int, _c_void_p]),
}

_lib: Optional[ctypes.CDLL] = None


class PaError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed: {status_str(status)} ({status}): {detail}")


def load() -> ctypes.CDLL:
    """Load libpa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        lib = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions the headers in include/ declare."""
    names = set()
    for h in sorted(INCLUDE.glob("*.h")):
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return sorted(names)


def status_str(status: int) -> str:
    return load().pa_status_str(status).decode()


def last_error() -> str:
    return load().pa_last_error().decode()


def abi_version() -> int:
    return load().pa_abi_version()


def _check(status: int, func: str) -> None:
    if status != 0:
        raise PaError(status, func, last_error())


def _dev(t: torch.Tensor, name: str, dtype=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _pool_shape(k_pool, v_pool) -> Tuple[int, int, int, int]:
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("k_pool and v_pool must both be [num_blocks][num_kv_heads][block_size][head_dim]")
    return tuple(k_pool.shape)


def _meta(block_tables, context_lens, B):
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    if context_lens.shape != (B,):
        raise ValueError("context_lens must be [num_seqs]")
    return block_tables.shape[1]


def pa_cache_write(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                   stream=None) -> None:
    """Store each sequence's newest token (position context_lens[s]-1) into its
    block slot, in place.  See pa_cache_write in include/pa.h."""
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool), ("k_new", k_new), ("v_new", v_new)):
        _dev(t, n)
    NB, Hkv, bs, d = _pool_shape(k_pool, v_pool)
    if k_new.dim() != 3 or k_new.shape[1:] != (Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    if not (k_pool.dtype == v_pool.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("pools and new rows must share one dtype")
    B = k_new.shape[0]
    MB = _meta(block_tables, context_lens, B)
    st = load().pa_cache_write(k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
                               v_new.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
                               B, Hkv, d, bs, MB, NB, _DTYPES.get(k_pool.dtype, -1),
                               _stream(k_pool.device, stream))
    _check(st, "pa_cache_write")


def _flags(shared_kv: bool, valu_only: bool) -> int:
    return (PA_FLAG_SHARED_KV if shared_kv else 0) | (PA_FLAG_VALU_ONLY if valu_only else 0)


def _decode_args(q, k_pool, v_pool, block_tables, context_lens, scale, out):
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    NB, Hkv, bs, d = _pool_shape(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != d:
        raise ValueError("q must be [num_seqs][num_heads][head_dim]")
    if not (q.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("q and the pools must share one dtype")
    B, Hq, _ = q.shape
    MB = _meta(block_tables, context_lens, B)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        raise TypeError("scale is required (usually 1/sqrt(head_dim), as an fp32 value)")
    return out, (B, Hq, Hkv, d, bs, MB, NB), float(scale)


def pa_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor,
              scale: float, out: Optional[torch.Tensor] = None,
              shared_kv: bool = False, valu_only: bool = False, stream=None) -> torch.Tensor:
    """Single-pass paged decode attention; returns ``out`` [num_seqs][num_heads][head_dim].
    ``shared_kv``: some blocks appear in several sequences' tables (keeps K/V
    loads cached instead of streaming); results are identical either way.
    ``valu_only``: grouped heads on the vector ALUs instead of the matrix
    cores (cross-checks and measurement)."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    st = load().pa_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                          block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, d, bs,
                          MB, NB, scale, _DTYPES.get(q.dtype, -1),
                          _flags(shared_kv, valu_only), _stream(q.device, stream))
    _check(st, "pa_decode")
    return out


def pa_decode_splitk_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int,
                                     max_context_len: int, partition_size: int) -> int:
    return int(load().pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim,
                                                       max_context_len, partition_size))


def pa_decode_splitk(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor,
                     partition_size: int, max_context_len: int,
                     scale: float, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, shared_kv: bool = False,
                     valu_only: bool = False, stream=None) -> torch.Tensor:
    """Split-K paged decode attention (partition pass + reduce pass)."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    need = pa_decode_splitk_workspace_bytes(B, Hq, d, max_context_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pa_decode_splitk(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(),
                                 v_pool.data_ptr(), block_tables.data_ptr(),
                                 context_lens.data_ptr(), B, Hq, Hkv, d, bs, MB, NB, scale,
                                 _DTYPES.get(q.dtype, -1), int(partition_size),
                                 int(max_context_len), workspace.data_ptr(), ws_bytes,
                                 _flags(shared_kv, valu_only), _stream(q.device, stream))
    _check(st, "pa_decode_splitk")
    return out


def _new_rows(k_new, v_new, k_pool, B, Hkv, d):
    _dev(k_new, "k_new", k_pool.dtype)
    _dev(v_new, "v_new", k_pool.dtype)
    if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")


def pa_write_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                    k_new: torch.Tensor, v_new: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, scale: float,
                    out: Optional[torch.Tensor] = None, shared_kv: bool = False,
                    valu_only: bool = False, stream=None) -> torch.Tensor:
    """One decode step: the new token's write (as pa_cache_write), then
    pa_decode, in one call.  See pa_write_decode in include/pa.h."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    _new_rows(k_new, v_new, k_pool, B, Hkv, d)
    st = load().pa_write_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(),
                                v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, d,
                                bs, MB, NB, scale, _DTYPES.get(q.dtype, -1),
                                _flags(shared_kv, valu_only), _stream(q.device, stream))
    _check(st, "pa_write_decode")
    return out


def pa_write_decode_splitk(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           k_new: torch.Tensor, v_new: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           partition_size: int, max_context_len: int, scale: float,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None, shared_kv: bool = False,
                           valu_only: bool = False, stream=None) -> torch.Tensor:
    """One decode step: the new token's write (as pa_cache_write), then
    pa_decode_splitk, in one call (the write runs in the plan's launch).
    See pa_write_decode_splitk in include/pa.h."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    _new_rows(k_new, v_new, k_pool, B, Hkv, d)
    need = pa_decode_splitk_workspace_bytes(B, Hq, d, max_context_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pa_write_decode_splitk(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, d, bs,
        MB, NB, scale, _DTYPES.get(q.dtype, -1), int(partition_size), int(max_context_len),
        workspace.data_ptr(), ws_bytes, _flags(shared_kv, valu_only), _stream(q.device, stream))
    _check(st, "pa_write_decode_splitk")
    return out


def pa_decode_splitk_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor,
                             partition_size: int, max_context_len: int, scale: float,
                             out: Optional[torch.Tensor] = None, shared_kv: bool = False,
                             valu_only: bool = False, stream=None) -> torch.Tensor:
    """Split-K paged decode without a workspace argument: the partials live in
    the library's static device scratch (PA_NOALLOC_SCRATCH_BYTES); for callers
    that cannot allocate.  See pa_decode_splitk_noalloc in include/pa.h."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    st = load().pa_decode_splitk_noalloc(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(),
                                         v_pool.data_ptr(), block_tables.data_ptr(),
                                         context_lens.data_ptr(), B, Hq, Hkv, d, bs, MB, NB,
                                         scale, _DTYPES.get(q.dtype, -1), int(partition_size),
                                         int(max_context_len), _flags(shared_kv, valu_only),
                                         _stream(q.device, stream))
    _check(st, "pa_decode_splitk_noalloc")
    return out


def _contiguous_shape(k_cache, v_cache) -> Tuple[int, int, int, int]:
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must both be "
                         "[num_seqs][num_kv_heads][max_len][head_dim]")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache must share one dtype")
    return tuple(k_cache.shape)


def pa_cache_write_contiguous(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                              v_new: torch.Tensor, context_lens: torch.Tensor,
                              stream=None) -> None:
    """Store each sequence's newest token (row context_lens[s]-1) into its
    region of a contiguous cache, in place.  See pa_cache_write_contiguous in
    include/pa.h."""
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        _dev(t, n)
    B, Hkv, max_len, d = _contiguous_shape(k_cache, v_cache)
    if k_new.shape != (B, Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs][num_kv_heads][head_dim]")
    if not (k_cache.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("caches and new rows must share one dtype")
    _dev(context_lens, "context_lens", torch.int32)
    if context_lens.shape != (B,):
        raise ValueError("context_lens must be [num_seqs]")
    st = load().pa_cache_write_contiguous(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(),
                                          v_new.data_ptr(), context_lens.data_ptr(), B, Hkv, d,
                                          max_len, _DTYPES.get(k_cache.dtype, -1),
                                          _stream(k_cache.device, stream))
    _check(st, "pa_cache_write_contiguous")


def pa_decode_contiguous(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         context_lens: torch.Tensor, scale: float, partition_size: int = 0,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, valu_only: bool = False,
                         stream=None) -> torch.Tensor:
    """Decode attention over a contiguous cache, k_cache and v_cache
    [num_seqs][num_kv_heads][max_len][head_dim], with no block table:
    ``partition_size`` 0 for one pass, else split-K with that partition.
    See pa_decode_contiguous in include/pa.h."""
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, n)
    B, Hkv, max_len, d = _contiguous_shape(k_cache, v_cache)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != d:
        raise ValueError("q must be [num_seqs][num_heads][head_dim] with k_cache's num_seqs "
                         "and head_dim")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    _dev(context_lens, "context_lens", torch.int32)
    if context_lens.shape != (B,):
        raise ValueError("context_lens must be [num_seqs]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if scale is None:
        raise TypeError("scale is required (usually 1/sqrt(head_dim), as an fp32 value)")
    Hq = q.shape[1]
    ws_ptr, ws_bytes = None, 0
    if partition_size:
        need = pa_decode_splitk_workspace_bytes(B, Hq, d, max_len, partition_size)
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        _dev(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = load().pa_decode_contiguous(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, d,
                                     max_len, float(scale), _DTYPES.get(q.dtype, -1),
                                     int(partition_size), ws_ptr, ws_bytes,
                                     _flags(False, valu_only), _stream(q.device, stream))
    _check(st, "pa_decode_contiguous")
    return out


def pa_decode_shared_prefix_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int,
                                            max_context_len: int, partition_size: int,
                                            num_groups: int) -> int:
    return int(load().pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_heads, head_dim, max_context_len, partition_size, num_groups))


def pa_decode_shared_prefix(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            seq_group: torch.Tensor, group_prefix_len: torch.Tensor,
                            max_group_size: int, partition_size: int, max_context_len: int,
                            scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, shared_kv: bool = False,
                            stream=None) -> torch.Tensor:
    """Decode for groups of sequences sharing a prompt's blocks; see
    pa_decode_shared_prefix in include/pa.h.  ``seq_group`` [num_seqs] int32
    (-1: no group), ``group_prefix_len`` [num_groups] int32."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    _dev(seq_group, "seq_group", torch.int32)
    _dev(group_prefix_len, "group_prefix_len", torch.int32)
    if seq_group.shape != (B,) or group_prefix_len.dim() != 1:
        raise ValueError("seq_group must be [num_seqs] and group_prefix_len [num_groups]")
    G = group_prefix_len.shape[0]
    need = pa_decode_shared_prefix_workspace_bytes(B, Hq, d, max_context_len, partition_size, G)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pa_decode_shared_prefix(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), seq_group.data_ptr(),
        group_prefix_len.data_ptr() if G else None, B, Hq, Hkv, d, bs, MB, NB, scale,
        _DTYPES.get(q.dtype, -1), G, int(max_group_size), int(partition_size),
        int(max_context_len), workspace.data_ptr(), ws_bytes,
        PA_FLAG_SHARED_KV if shared_kv else 0, _stream(q.device, stream))
    _check(st, "pa_decode_shared_prefix")
    return out


def pa_write_decode_shared_prefix(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  k_new: torch.Tensor, v_new: torch.Tensor,
                                  block_tables: torch.Tensor, context_lens: torch.Tensor,
                                  seq_group: torch.Tensor, group_prefix_len: torch.Tensor,
                                  max_group_size: int, partition_size: int,
                                  max_context_len: int, scale: float,
                                  out: Optional[torch.Tensor] = None,
                                  workspace: Optional[torch.Tensor] = None,
                                  shared_kv: bool = False, stream=None) -> torch.Tensor:
    """One decode step with shared prompts: the new token's write, then
    pa_decode_shared_prefix, in one call.  See pa_write_decode_shared_prefix
    in include/pa.h."""
    out, (B, Hq, Hkv, d, bs, MB, NB), scale = _decode_args(q, k_pool, v_pool, block_tables,
                                                           context_lens, scale, out)
    _new_rows(k_new, v_new, k_pool, B, Hkv, d)
    _dev(seq_group, "seq_group", torch.int32)
    _dev(group_prefix_len, "group_prefix_len", torch.int32)
    if seq_group.shape != (B,) or group_prefix_len.dim() != 1:
        raise ValueError("seq_group must be [num_seqs] and group_prefix_len [num_groups]")
    G = group_prefix_len.shape[0]
    need = pa_decode_shared_prefix_workspace_bytes(B, Hq, d, max_context_len, partition_size, G)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pa_write_decode_shared_prefix(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), seq_group.data_ptr(),
        group_prefix_len.data_ptr() if G else None, B, Hq, Hkv, d, bs, MB, NB, scale,
        _DTYPES.get(q.dtype, -1), G, int(max_group_size), int(partition_size),
        int(max_context_len), workspace.data_ptr(), ws_bytes,
        PA_FLAG_SHARED_KV if shared_kv else 0, _stream(q.device, stream))
    _check(st, "pa_write_decode_shared_prefix")
    return out


def pa_copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor,
                   stream=None) -> None:
    """Copy whole blocks of both pools: pairs int32 [n][2] (source,
    destination) on the device.  See pa_copy_blocks in include/pa.h."""
    for n, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(t, n)
    _dev(pairs, "pairs", torch.int32)
    NB, Hkv, bs, d = _pool_shape(k_pool, v_pool)
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [num_pairs][2]")
    st = load().pa_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), pairs.data_ptr(),
                               pairs.shape[0], Hkv, d, bs, NB, _DTYPES.get(k_pool.dtype, -1),
                               _stream(k_pool.device, stream))
    _check(st, "pa_copy_blocks")


def pa_swap_blocks(dst_k: torch.Tensor, dst_v: torch.Tensor, src_k: torch.Tensor,
                   src_v: torch.Tensor, pairs, stream=None) -> None:
    """Move blocks between a device pool and a host pool (one of each);
    pairs [n][2] (source block, destination block) on the host."""
    import numpy as np
    if dst_k.shape[1:] != src_k.shape[1:] or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("pools must share [num_kv_heads][block_size][head_dim]")
    if dst_k.dtype != src_k.dtype:
        raise TypeError("pools must share one dtype")
    for t in (dst_k, dst_v, src_k, src_v):
        if not t.is_contiguous():
            raise ValueError("pools must be contiguous")
    if dst_k.device.type == src_k.device.type:
        raise ValueError("one pool must be on the host and one on the device")
    to_host = 1 if dst_k.device.type == "cpu" else 0
    dev = src_k.device if to_host else dst_k.device
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    block_bytes = dst_k[0].numel() * dst_k.element_size()
    st = load().pa_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), src_k.data_ptr(),
                               src_v.data_ptr(), pr.ctypes.data, pr.shape[0], dst_k.shape[0],
                               src_k.shape[0], block_bytes, to_host, _stream(dev, stream))
    _check(st, "pa_swap_blocks")


def pa_read_probe(buf: torch.Tensor, tile_bytes: int, tile_order: torch.Tensor,
                  sink: torch.Tensor, stream=None) -> None:
    """Read the tiles of ``buf`` named by ``tile_order`` (int32, device) with
    the decode kernels' loads; a measurement aid (see include/pa.h)."""
    _dev(buf, "buf")
    _dev(tile_order, "tile_order")
    _dev(sink, "sink")
    if tile_order.dtype != torch.int32 or tile_order.dim() != 1:
        raise TypeError("tile_order must be a 1-D int32 tensor")
    nbytes = buf.numel() * buf.element_size()
    if tile_bytes <= 0 or tile_bytes % 4096 or nbytes < tile_bytes:
        raise ValueError("tile_bytes must be a positive multiple of 4096 within the buffer")
    st = load().pa_read_probe(buf.data_ptr(), tile_bytes, tile_order.data_ptr(),
                              tile_order.numel(), sink.data_ptr(), _stream(buf.device, stream))
    _check(st, "pa_read_probe")


def pa_device_memory(device: int = 0) -> Tuple[int, int]:
    """(memory bus width in bits, peak memory clock in kHz) as the HIP runtime
    reports them for ``device``; a measurement aid (see include/pa.h)."""
    bw, clk = ctypes.c_int(0), ctypes.c_int(0)
    _check(load().pa_device_memory(device, ctypes.byref(bw), ctypes.byref(clk)), "pa_device_memory")
    return bw.value, clk.value


def pa_check_inputs_host(block_tables, context_lens, block_size: int, num_blocks: int,
                         check_write_targets: bool = False) -> Tuple[bool, int, str]:
    """Validate host copies of the tables and lengths.  Returns
    (ok, first bad sequence or -1, message)."""
    import numpy as np
    tb = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    ln = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if tb.ndim != 2 or ln.shape != (tb.shape[0],):
        raise ValueError("block_tables must be [B][MB] and context_lens [B]")
    bad = _c_int(-1)
    st = load().pa_check_inputs_host(tb.ctypes.data, ln.ctypes.data, tb.shape[0], block_size,
                                     tb.shape[1], num_blocks, int(bool(check_write_targets)),
                                     ctypes.byref(bad))
    return st == 0, bad.value, last_error()
