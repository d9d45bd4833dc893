"""Python binding of libpagedkv.so — argument marshalling only.

Every function here checks tensor placement and dtypes, turns tensors into pointers and
sizes, and calls the C ABI declared in include/pagedkv.h with the same name (minus the
``pkv_`` prefix).  All computation happens in the library's HIP kernels (or, for the
block allocator, in its C++ host code).  There is no fallback: if the library is not
built, every call raises.

PyTorch provides device memory and streams only.  torch is imported before the library
is loaded so that the library binds to the HIP runtime torch already mapped (both carry
the SONAME libamdhip64.so.7); ``_check_single_hip_runtime`` verifies that only one
runtime is mapped into the process.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

__all__ = [
    "PagedKVError", "lib", "library_path", "exported_symbols",
    "F32", "BF16", "FP8_E4M3FN",
    "allocate_kv_pool", "paged_attention_workspace_size", "paged_attention_default_splits",
    "paged_attention_decode",
    "paged_attention_split", "paged_attention_reduce", "paged_decode_step", "paged_decode_step_split",
    "contiguous_attention_decode", "paged_attention_grouped_workspace_size", "paged_attention_decode_grouped",
    "paged_decode_step_grouped", "paged_attention_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "kv_cache_write", "copy_blocks",
    "build_slot_mapping", "BlockAllocator", "abi_version", "set_launch_events", "apply_append",
    "paged_attention_prefill", "paged_attention_prefill_workspace_size", "FEW_QUERY_COLUMNS",
    "allocate_host_pool", "swap_blocks", "VmmPool",
]

F32, BF16, FP8_E4M3FN = 0, 1, 2
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "OUT_OF_BLOCKS", 4: "UNKNOWN_SEQ",
           5: "HIP_ERROR"}
_PKG = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the library to load instead (the host sanitizer build of
# the allocator, which has only the host entry points; calls to any other entry point then
# raise AttributeError).
_LIB_OVERRIDE = os.environ.get("PKV_LIBRARY")
library_path = _LIB_OVERRIDE or os.path.join(_PKG, "libpagedkv.so")


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = _STATUS.get(status, str(status))


_lib = None
_lock = threading.Lock()
_c_int, _c_i64, _c_f, _c_p, _c_sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_DECODE_ARGS = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                _c_int, _c_f, _c_f, _c_f, _c_int, _c_int, _c_int, _c_p, _c_sz, _c_p, _c_p]
_STEP_ARGS = [_c_p] * 8 + [_c_int] * 7 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_sz, _c_p, _c_p]
_SIGNATURES = {
    "pkv_abi_version": ([], _c_int),
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_paged_attention_workspace_size": ([_c_int] * 8 + [ctypes.POINTER(_c_sz)], _c_int),
    "pkv_paged_attention_default_splits": ([_c_int] * 4 + [ctypes.POINTER(_c_int)], _c_int),
    "pkv_paged_attention_decode": (_DECODE_ARGS, _c_int),
    "pkv_paged_attention_split": (_DECODE_ARGS, _c_int),
    "pkv_paged_attention_reduce": (_DECODE_ARGS, _c_int),
    "pkv_paged_attention_decode_noalloc": ([_c_p] * 6 + [_c_int] * 7 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_p],
                                           _c_int),
    "pkv_paged_attention_grouped_workspace_size": ([_c_int] * 9 + [ctypes.POINTER(_c_sz)], _c_int),
    "pkv_paged_attention_decode_grouped": ([_c_p] * 9 + [_c_int] * 7 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_sz, _c_p],
                                           _c_int),
    "pkv_paged_decode_step_grouped": ([_c_p] * 11 + [_c_int] * 7 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_sz, _c_p],
                                      _c_int),
    "pkv_alloc_prefix_groups": ([_c_p, _c_p, _c_int, _c_int, _c_p, _c_p, _c_p], _c_int),
    "pkv_contiguous_attention_decode": ([_c_p] * 6 + [_c_int] * 7 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_sz, _c_p],
                                        _c_int),
    "pkv_paged_decode_step": (_STEP_ARGS, _c_int),
    "pkv_set_launch_events": ([_c_p, _c_p], _c_int),
    "pkv_apply_append": ([_c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_p], _c_int),
    "pkv_paged_decode_step_split": (_STEP_ARGS, _c_int),
    "pkv_paged_attention_prefill": ([_c_p] * 7 + [_c_int] * 9 + [_c_f] * 3 + [_c_int] * 3 + [_c_p, _c_sz, _c_p, _c_p],
                                    _c_int),
    "pkv_paged_attention_prefill_workspace_size": ([_c_int] * 9 + [ctypes.POINTER(_c_sz)], _c_int),
    "pkv_kv_cache_write": ([_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_int, _c_int, _c_f, _c_f, _c_p], _c_int),
    "pkv_copy_blocks": ([_c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_p], _c_int),
    "pkv_swap_blocks": ([_c_p, _c_p, _c_int, _c_p, _c_p, _c_int, _c_p] + [_c_int] * 5 + [_c_p], _c_int),
    "pkv_seq_swap": ([_c_p, _c_p, _c_i64, _c_p, _c_p], _c_int),
    "pkv_alloc_stats_get": ([_c_p, _c_p], _c_int),
    "pkv_vmm_create": ([_c_int, _c_int, _c_int, _c_sz, _c_sz], _c_p),
    "pkv_vmm_destroy": ([_c_p], None),
    "pkv_vmm_reserve": ([_c_p, _c_int, _c_int], _c_int),
    "pkv_vmm_release": ([_c_p, _c_int], _c_int),
    "pkv_vmm_k_base": ([_c_p], _c_p),
    "pkv_vmm_v_base": ([_c_p], _c_p),
    "pkv_vmm_num_blocks": ([_c_p], _c_int),
    "pkv_vmm_seq_first_block": ([_c_p, _c_int], _c_int),
    "pkv_vmm_mapped_blocks": ([_c_p, _c_int], _c_int),
    "pkv_vmm_mapped_bytes": ([_c_p], _c_sz),
    "pkv_vmm_page_bytes": ([_c_p], _c_sz),
    "pkv_alloc_create": ([_c_int, _c_int, _c_p], _c_p),
    "pkv_alloc_destroy": ([_c_p], None),
    "pkv_seq_create": ([_c_p, _c_i64, _c_i64, _c_p], _c_int),
    "pkv_seq_fork": ([_c_p, _c_i64, _c_i64, _c_i64], _c_int),
    "pkv_seq_extend": ([_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p], _c_int),
    "pkv_seq_append": ([_c_p, _c_p, _c_int, _c_p, _c_p, _c_p], _c_int),
    "pkv_seq_free": ([_c_p, _c_i64], _c_int),
    "pkv_alloc_block_tables": ([_c_p, _c_p, _c_int, _c_int, _c_p, _c_p], _c_int),
    "pkv_alloc_shared_prefix_blocks": ([_c_p, _c_p, _c_int, _c_p], _c_int),
    "pkv_alloc_num_free": ([_c_p], _c_int),
    "pkv_alloc_num_blocks": ([_c_p], _c_int),
    "pkv_alloc_block_size": ([_c_p], _c_int),
    "pkv_alloc_refcount": ([_c_p, _c_int], _c_int),
    "pkv_alloc_num_seqs": ([_c_p], _c_int),
    "pkv_seq_info": ([_c_p, _c_i64, _c_p, _c_p], _c_int),
    "pkv_alloc_free_list": ([_c_p, _c_p, _c_int], _c_int),
    "pkv_build_slot_mapping": ([_c_p, _c_p, _c_int, _c_int, _c_int, _c_p], _c_int),
}
exported_symbols = tuple(_SIGNATURES)


def _check_single_hip_runtime():
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"more than one HIP runtime mapped into this process: {sorted(real)}")


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(library_path):
                raise RuntimeError(f"{library_path} is not built; run `python -m paged_kv_cache_329_amd.build`")
            handle = ctypes.CDLL(library_path)
            for name, (args, res) in _SIGNATURES.items():
                if _LIB_OVERRIDE and not hasattr(handle, name):
                    continue
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _check_single_hip_runtime()
            _lib = handle
    return _lib


def abi_version() -> int:
    return lib().pkv_abi_version()


def _check(status: int):
    if status != 0:
        raise PagedKVError(status, lib().pkv_last_error().decode(errors="replace"))


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t}")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _np(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def allocate_kv_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                     dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Uninitialised pool tensor [num_blocks, num_kv_heads, block_size * head_dim].

    The innermost block_size * head_dim elements of each (block, head) are in the tiled
    layout of include/pagedkv.h, not row-major [block_size, head_dim].
    """
    return torch.empty((num_blocks, num_kv_heads, block_size * head_dim), dtype=dtype, device=device)


def _pool_dims(k_cache: torch.Tensor, head_dim: int):
    if k_cache.dim() != 3 or k_cache.shape[2] % head_dim:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size * head_dim]")
    return k_cache.shape[0], k_cache.shape[1], k_cache.shape[2] // head_dim


def paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                   q_dtype, kv_dtype, num_splits=0) -> int:
    out = _c_sz(0)
    _check(lib().pkv_paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                    block_size, q_dtype, kv_dtype, num_splits,
                                                    ctypes.byref(out)))
    return out.value


def paged_attention_default_splits(head_dim, block_size, q_dtype, kv_dtype) -> int:
    """Split count used for num_splits=0 on the current device (queries the device)."""
    out = _c_int(0)
    _check(lib().pkv_paged_attention_default_splits(head_dim, block_size, q_dtype, kv_dtype,
                                                    ctypes.byref(out)))
    return out.value


_ws_cache: dict = {}


def _workspace(nbytes: int, device, stream_handle: int) -> torch.Tensor:
    # One cached workspace per (device, stream): calls on one stream run in order.
    key = (str(device), stream_handle)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _prefix_arg(t, n: int):
    """Device address of a shared_prefix_blocks hint (contiguous int32 [n] on the device), or None."""
    if t is None:
        return None
    if t.dtype != torch.int32 or t.shape != (n,) or not t.is_contiguous():
        raise ValueError("shared_prefix_blocks must be a contiguous int32 [num_seqs] tensor")
    return _dev(t, "shared_prefix_blocks")


def _decode_call(fn_name, out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                 v_scale, num_splits, workspace, stream, shared_prefix_blocks):
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim] of one dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_cache, D)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    qd, kd = _dtype_code(q.dtype), _dtype_code(k_cache.dtype)
    st = _stream(stream)
    if workspace is None:
        nbytes = paged_attention_workspace_size(B, Hq, Hkv, D, bs, qd, kd, num_splits)
        workspace = _workspace(nbytes, q.device, st)
    ptrs = [_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens")]
    _check(getattr(lib(), fn_name)(*ptrs, B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                                   float(scale), float(k_scale), float(v_scale), qd, kd,
                                   int(num_splits), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(),
                                   _prefix_arg(shared_prefix_blocks, B), st))
    return out


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None,
                           shared_prefix_blocks=None):
    """Decode attention through block tables (both phases); see pkv_paged_attention_decode.
    shared_prefix_blocks: optional device int32 [num_seqs], the leading blocks of each sequence
    that other sequences also read (BlockAllocator.shared_prefix_blocks); those are read
    through the caches, the rest streamed.  The output bits do not depend on it."""
    return _decode_call("pkv_paged_attention_decode", out, q, k_cache, v_cache, block_tables,
                        context_lens, scale, k_scale, v_scale, num_splits, workspace, stream,
                      shared_prefix_blocks)


def paged_attention_split(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                          k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None,
                          shared_prefix_blocks=None):
    """Phase 1 only (streams K/V, writes finished heads and partials)."""
    return _decode_call("pkv_paged_attention_split", out, q, k_cache, v_cache, block_tables,
                        context_lens, scale, k_scale, v_scale, num_splits, workspace, stream,
                      shared_prefix_blocks)


def paged_attention_reduce(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None,
                           shared_prefix_blocks=None):
    """Phase 2 only (merges partials); same arguments and workspace as phase 1."""
    return _decode_call("pkv_paged_attention_reduce", out, q, k_cache, v_cache, block_tables,
                        context_lens, scale, k_scale, v_scale, num_splits, workspace, stream,
                      shared_prefix_blocks)


NOALLOC_SCRATCH_BYTES = 48 << 20


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=1.0,
                                   v_scale=1.0, num_splits=0, stream=None, shared_prefix_blocks=None):
    """pkv_paged_attention_decode_noalloc: decode attention with the library's own scratch in
    place of a workspace; allocates nothing (here or in the library)."""
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim] of one dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_cache, D)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    _check(lib().pkv_paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), B, Hq, Hkv, D, bs, NB,
        block_tables.shape[1], float(scale), float(k_scale), float(v_scale), _dtype_code(q.dtype),
        _dtype_code(k_cache.dtype), int(num_splits), _prefix_arg(shared_prefix_blocks, B), _stream(stream)))
    return out


def paged_attention_grouped_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, q_dtype,
                                           kv_dtype, num_splits=0, max_blocks_per_seq=0) -> int:
    n = _c_sz(0)
    _check(lib().pkv_paged_attention_grouped_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                            q_dtype, kv_dtype, int(num_splits),
                                                            int(max_blocks_per_seq), ctypes.byref(n)))
    return n.value


def _group_args(groups, B):
    if len(groups) != 3:
        raise ValueError("groups must be (chunk_first, chunk_src, group_blocks)")
    for t in groups:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.shape != (B,):
            raise ValueError("chunk_first, chunk_src and group_blocks must be int32 [num_seqs] device tensors")
    return [_dev(t, "group array") for t in groups]


def paged_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, groups, scale,
                                   k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None):
    """Decode with prefix groups (pkv_paged_attention_decode_grouped): groups is the device
    triple (chunk_first, chunk_src, group_blocks) of BlockAllocator.prefix_groups."""
    return _grouped_call("pkv_paged_attention_decode_grouped", out, q, None, None, k_cache, v_cache, block_tables,
                         context_lens, groups, scale, k_scale, v_scale, num_splits, workspace, stream)


def paged_decode_step_grouped(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, groups, scale,
                              k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None):
    """The decode step with append, with prefix groups (pkv_paged_decode_step_grouped)."""
    return _grouped_call("pkv_paged_decode_step_grouped", out, q, k_new, v_new, k_cache, v_cache, block_tables,
                         context_lens, groups, scale, k_scale, v_scale, num_splits, workspace, stream)


def _grouped_call(fn_name, out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, groups, scale,
                  k_scale, v_scale, num_splits, workspace, stream):
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim] of one dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_cache, D)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    qd, kd = _dtype_code(q.dtype), _dtype_code(k_cache.dtype)
    st = _stream(stream)
    if workspace is None:
        workspace = _workspace(paged_attention_grouped_workspace_size(B, Hq, Hkv, D, bs, qd, kd, num_splits,
                                                                      block_tables.shape[1]), q.device, st)
    ptrs = [_dev(out, "out"), _dev(q, "q")]
    if k_new is not None:
        if k_new.shape != (B, Hkv, D) or v_new.shape != k_new.shape or k_new.dtype != q.dtype or v_new.dtype != q.dtype:
            raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim] of q's dtype")
        ptrs += [_dev(k_new, "k_new"), _dev(v_new, "v_new")]
    ptrs += [_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
             _dev(context_lens, "context_lens")] + _group_args(groups, B)
    _check(getattr(lib(), fn_name)(*ptrs, B, Hq, Hkv, D, bs, NB, block_tables.shape[1], float(scale), float(k_scale),
                                   float(v_scale), qd, kd, int(num_splits), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), st))
    return out


def contiguous_attention_decode(out, q, k_base, v_base, seq_first_block, context_lens, max_blocks_per_seq,
                                scale, k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None):
    """Decode attention over contiguous per-sequence placement (pkv_contiguous_attention_decode):
    logical block j of sequence s is pool block seq_first_block[s] + j; no block table."""
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim] of one dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_base, D)
    if v_base.shape != k_base.shape or v_base.dtype != k_base.dtype:
        raise ValueError("v_base must match k_base")
    if seq_first_block.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("seq_first_block and context_lens must be int32")
    if seq_first_block.shape != (B,) or context_lens.shape != (B,):
        raise ValueError("seq_first_block and context_lens must be [num_seqs]")
    qd, kd = _dtype_code(q.dtype), _dtype_code(k_base.dtype)
    st = _stream(stream)
    if workspace is None:
        workspace = _workspace(paged_attention_workspace_size(B, Hq, Hkv, D, bs, qd, kd, num_splits), q.device, st)
    _check(lib().pkv_contiguous_attention_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_base, "k_base"), _dev(v_base, "v_base"),
        _dev(seq_first_block, "seq_first_block"), _dev(context_lens, "context_lens"), B, Hq, Hkv, D, bs, NB,
        int(max_blocks_per_seq), float(scale), float(k_scale), float(v_scale), qd, kd, int(num_splits),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), st))
    return out


# pkv_paged_attention_prefill takes the few-query path (split over the keys, then a merge)
# when max_query_len * (num_q_heads / num_kv_heads) is at most this, query tiles otherwise.
FEW_QUERY_COLUMNS = 32


def paged_attention_prefill_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                           q_dtype, kv_dtype, max_query_len, num_splits=0) -> int:
    n = _c_sz(0)
    _check(lib().pkv_paged_attention_prefill_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                            block_size, q_dtype, kv_dtype, int(max_query_len),
                                                            int(num_splits), ctypes.byref(n)))
    return n.value


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                            max_query_len, scale, k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None,
                            stream=None, shared_prefix_blocks=None):
    """Causal multi-query attention (pkv_paged_attention_prefill): sequence s's queries are
    q rows query_start[s] .. query_start[s+1]-1, its last tokens, each attending to every
    token up to its own position.  q / out are [num_q_tokens, Hq, D].  When none is given, a
    workspace is made (and cached per stream): the few-query path needs one, and with one the
    tile path launches its tiles longest first."""
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_q_tokens, num_q_heads, head_dim] of one dtype")
    T, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_cache, D)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or query_start.dtype != torch.int32:
        raise TypeError("block_tables, context_lens and query_start must be int32")
    B = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.dim() != 1 or query_start.shape != (B + 1,):
        raise ValueError("block_tables [num_seqs, max_blocks], context_lens [num_seqs], query_start [num_seqs+1]")
    qd, kd = _dtype_code(q.dtype), _dtype_code(k_cache.dtype)
    st = _stream(stream)
    if workspace is None:
        nbytes = paged_attention_prefill_workspace_size(B, Hq, Hkv, D, bs, qd, kd, max_query_len, num_splits)
        workspace = _prefill_workspace(nbytes, q.device, st) if nbytes else None
    ptrs = [_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
            _dev(query_start, "query_start")]
    _check(lib().pkv_paged_attention_prefill(*ptrs, B, T, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                                             int(max_query_len), float(scale), float(k_scale),
                                             float(v_scale), qd, kd, int(num_splits),
                                             _dev(workspace, "workspace") if workspace is not None else None,
                                             workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                             _prefix_arg(shared_prefix_blocks, B), st))
    return out


_prefill_ws_cache: dict = {}


def _prefill_workspace(nbytes: int, device, stream_handle: int) -> torch.Tensor:
    key = (str(device), stream_handle)
    ws = _prefill_ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _prefill_ws_cache[key] = ws
    return ws


def _step_call(fn_name, out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
               k_scale, v_scale, num_splits, workspace, stream, shared_prefix_blocks):
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [num_seqs, num_q_heads, head_dim] of one dtype")
    B, Hq, D = q.shape
    NB, Hkv, bs = _pool_dims(k_cache, D)
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must match k_cache")
    if k_new.shape != (B, Hkv, D) or v_new.shape != k_new.shape or k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim] of q's dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    qd, kd = _dtype_code(q.dtype), _dtype_code(k_cache.dtype)
    st = _stream(stream)
    if workspace is None:
        nbytes = paged_attention_workspace_size(B, Hq, Hkv, D, bs, qd, kd, num_splits)
        workspace = _workspace(nbytes, q.device, st)
    ptrs = [_dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
            _dev(context_lens, "context_lens")]
    _check(getattr(lib(), fn_name)(*ptrs, B, Hq, Hkv, D, bs, NB, block_tables.shape[1],
                                   float(scale), float(k_scale), float(v_scale), qd, kd,
                                   int(num_splits), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(),
                                   _prefix_arg(shared_prefix_blocks, B), st))
    return out


def paged_decode_step(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                      k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None,
                      shared_prefix_blocks=None):
    """Decode step with append (pkv_paged_decode_step): stores every sequence's new token
    (k_new / v_new [num_seqs, Hkv, D], q's dtype) at position context_lens[s] - 1, then
    attends over all context_lens[s] tokens; the store is fused into the split pass."""
    return _step_call("pkv_paged_decode_step", out, q, k_new, v_new, k_cache, v_cache, block_tables,
                      context_lens, scale, k_scale, v_scale, num_splits, workspace, stream,
                      shared_prefix_blocks)


def paged_decode_step_split(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                            k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None,
                            shared_prefix_blocks=None):
    """Phase 1 of the decode step (append + split pass); phase 2 is paged_attention_reduce."""
    return _step_call("pkv_paged_decode_step_split", out, q, k_new, v_new, k_cache, v_cache, block_tables,
                      context_lens, scale, k_scale, v_scale, num_splits, workspace, stream,
                      shared_prefix_blocks)


def set_launch_events(start, stop):
    """The next split pass launched on this thread records these torch.cuda.Event objects
    around its own kernel (pkv_set_launch_events).  The events must already exist on the
    device: record each of them once beforehand."""
    _check(lib().pkv_set_launch_events(start.cuda_event if start is not None else None,
                                       stop.cuda_event if stop is not None else None))


def kv_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale=1.0, v_scale=1.0,
                   stream=None):
    """Store new tokens [T, Hkv, D] into their slots (quantising for an fp8 cache)."""
    if k_new.dim() != 3 or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must both be [num_tokens, num_kv_heads, head_dim]")
    T, Hkv, D = k_new.shape
    NB, Hkv_c, bs = _pool_dims(k_cache, D)
    if Hkv_c != Hkv or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("pool shape does not match the new tokens")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    _check(lib().pkv_kv_cache_write(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
                                    _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"), T, Hkv,
                                    D, bs, NB, _dtype_code(k_new.dtype), _dtype_code(k_cache.dtype),
                                    float(k_scale), float(v_scale), _stream(stream)))


def copy_blocks(k_cache, v_cache, block_mapping, head_dim: int, stream=None):
    """Copy whole blocks for copy-on-write; block_mapping is int32 [n, 2] of (src, dst)."""
    NB, Hkv, bs = _pool_dims(k_cache, head_dim)
    if block_mapping.dtype != torch.int32 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int32 [num_pairs, 2]")
    n = block_mapping.shape[0]
    _check(lib().pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                 _dev(block_mapping, "block_mapping") if n else None, n, Hkv,
                                 head_dim, bs, NB, _dtype_code(k_cache.dtype), _stream(stream)))


def allocate_host_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                       dtype: torch.dtype) -> torch.Tensor:
    """Pinned host pool [num_blocks, num_kv_heads, block_size * head_dim] (same layout as the
    device pool), for swapped-out sequences; the device reads and writes it directly."""
    return torch.empty((num_blocks, num_kv_heads, block_size * head_dim), dtype=dtype, pin_memory=True)


def _pool_ptr(t: torch.Tensor, name: str) -> int:
    # A device tensor, or a pinned host tensor (device-accessible at the same address).
    if isinstance(t, torch.Tensor) and not t.is_cuda:
        if not t.is_pinned():
            raise ValueError(f"{name} must be a device tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t.data_ptr()
    return _dev(t, name)


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, head_dim: int, stream=None):
    """Copy whole blocks between two pools of the same layout (pkv_swap_blocks): device <->
    pinned host for a swap.  block_mapping is int32 [n, 2] of (src, dst) on the device."""
    SNB, Hkv, bs = _pool_dims(src_k, head_dim)
    DNB, Hkv2, bs2 = _pool_dims(dst_k, head_dim)
    if (Hkv, bs) != (Hkv2, bs2) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools must share kv heads, block size and dtype")
    if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
        raise ValueError("V pools must match their K pools")
    if block_mapping.dtype != torch.int32 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int32 [num_pairs, 2]")
    n = block_mapping.shape[0]
    _check(lib().pkv_swap_blocks(_pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"), DNB,
                                 _pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"), SNB,
                                 _dev(block_mapping, "block_mapping") if n else None, n, Hkv, head_dim, bs,
                                 _dtype_code(src_k.dtype), _stream(stream)))


def apply_append(block_tables, context_lens, slot_mapping, block_size: int, num_blocks: int, stream=None):
    """Mirror a decode step's append on device tables / lengths (pkv_apply_append).
    slot_mapping may be a device tensor or a pinned host tensor (read by the kernel)."""
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or slot_mapping.dtype != torch.int64:
        raise TypeError("block_tables / context_lens must be int32 and slot_mapping int64")
    n = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != n or slot_mapping.shape != (n,):
        raise ValueError("block_tables [n, max_blocks], context_lens [n], slot_mapping [n]")
    if not slot_mapping.is_cuda and not slot_mapping.is_pinned():
        raise ValueError("slot_mapping must be a device tensor or a pinned host tensor")
    if not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous")
    _check(lib().pkv_apply_append(_dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
                                  slot_mapping.data_ptr(), n, block_tables.shape[1], block_size,
                                  num_blocks, _stream(stream)))


def build_slot_mapping(block_tables, lens, block_size: int) -> np.ndarray:
    """Host slot mapping of whole sequences (pkv_build_slot_mapping)."""
    t = _np(block_tables, np.int32)
    ln = _np(lens, np.int32)
    out = np.empty(int(ln.sum()), dtype=np.int64)
    _check(lib().pkv_build_slot_mapping(t.ctypes.data, ln.ctypes.data, len(ln), t.shape[1],
                                        block_size, out.ctypes.data))
    return out


class _DeviceArray:
    """A device address range described through __cuda_array_interface__, so that torch can
    view memory the library mapped (the tensor does not own it)."""

    def __init__(self, ptr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (int(ptr), False),
                                         "version": 2, "strides": None}


_RAW = {torch.float32: ("<f4", torch.float32), torch.bfloat16: ("<i2", torch.bfloat16),
        torch.float8_e4m3fn: ("|u1", torch.float8_e4m3fn)}


class VmmPool:
    """K/V pools in contiguous virtual memory mapped on demand (pkv_vmm_*).

    ``k`` and ``v`` are [num_blocks, Hkv, bs * D] views of the reserved ranges, in the pool
    layout; sequence ``seq``'s logical block j is block ``first_block(seq) + j``.  Only the
    blocks made resident with ``reserve`` (and block 0) may be read or written.
    """

    def __init__(self, max_seqs: int, max_blocks_per_seq: int, num_kv_heads: int, block_size: int,
                 head_dim: int, dtype: torch.dtype, device: int = 0, page_bytes: int = 0):
        eb = torch.empty((), dtype=dtype).element_size()
        self.block_bytes = num_kv_heads * block_size * head_dim * eb
        h = lib().pkv_vmm_create(device, max_seqs, max_blocks_per_seq, self.block_bytes, page_bytes)
        if not h:
            raise PagedKVError(2, lib().pkv_last_error().decode(errors="replace"))
        self._h = h
        nb = lib().pkv_vmm_num_blocks(h)
        typestr, tdt = _RAW[dtype]
        shape = (nb, num_kv_heads, block_size * head_dim)
        with torch.cuda.device(device):
            self.k = torch.as_tensor(_DeviceArray(lib().pkv_vmm_k_base(h), shape, typestr), device=f"cuda:{device}").view(tdt)
            self.v = torch.as_tensor(_DeviceArray(lib().pkv_vmm_v_base(h), shape, typestr), device=f"cuda:{device}").view(tdt)

    def reserve(self, seq: int, num_blocks: int):
        _check(lib().pkv_vmm_reserve(self._h, seq, num_blocks))

    def release(self, seq: int):
        _check(lib().pkv_vmm_release(self._h, seq))

    def first_block(self, seq: int) -> int:
        return lib().pkv_vmm_seq_first_block(self._h, seq)

    def mapped_blocks(self, seq: int) -> int:
        return lib().pkv_vmm_mapped_blocks(self._h, seq)

    @property
    def mapped_bytes(self) -> int:
        return lib().pkv_vmm_mapped_bytes(self._h)

    @property
    def page_bytes(self) -> int:
        return lib().pkv_vmm_page_bytes(self._h)

    def close(self):
        if getattr(self, "_h", None):
            self.k = self.v = None
            lib().pkv_vmm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass


class _AllocStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("num_blocks", "free_blocks", "used_blocks", "shared_blocks",
                                              "logical_blocks", "tokens", "stored_tokens", "num_seqs")]


class BlockAllocator:
    """Host block allocator (pkv_alloc_*): free list, refcounts, copy-on-write decisions."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        order = None if free_order is None else _np(free_order, np.int32)
        self._order = order
        h = lib().pkv_alloc_create(num_blocks, block_size, None if order is None else order.ctypes.data)
        if not h:
            raise PagedKVError(1, lib().pkv_last_error().decode(errors="replace"))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None):
            lib().pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_create(self, seq_id: int, length: int) -> np.ndarray:
        slots = np.empty(max(length, 0), dtype=np.int64)
        _check(lib().pkv_seq_create(self._h, seq_id, length, slots.ctypes.data if length > 0 else None))
        return slots

    def fork(self, parent: int, child: int, prefix_len: int):
        _check(lib().pkv_seq_fork(self._h, parent, child, prefix_len))

    def extend(self, seq_id: int, n: int):
        slots = np.empty(max(n, 0), dtype=np.int64)
        cow = np.empty((1, 2), dtype=np.int32)
        ncow = ctypes.c_int(0)
        _check(lib().pkv_seq_extend(self._h, seq_id, n, slots.ctypes.data if n > 0 else None,
                                    cow.ctypes.data, ctypes.byref(ncow)))
        return slots, cow[:ncow.value].copy()

    def append(self, seq_ids, slots_out=None, cow_out=None):
        """One token for each listed sequence -> (slots, copy-on-write pairs).

        slots_out (int64 [n]) and cow_out (int32 [>= n, 2]), if given, are filled in place
        (for example numpy views of pinned host tensors) and views of them are returned.
        """
        ids = _np(seq_ids, np.int64)
        n = len(ids)
        slots = np.empty(n, dtype=np.int64) if slots_out is None else slots_out
        cow = np.empty((max(n, 1), 2), dtype=np.int32) if cow_out is None else cow_out
        if slots.dtype != np.int64 or slots.shape[0] < n or not slots.flags.c_contiguous:
            raise ValueError("slots_out must be a contiguous int64 array of at least n entries")
        if cow.dtype != np.int32 or cow.shape[0] < max(n, 1) or not cow.flags.c_contiguous:
            raise ValueError("cow_out must be a contiguous int32 [>= n, 2] array")
        ncow = ctypes.c_int(0)
        _check(lib().pkv_seq_append(self._h, ids.ctypes.data, n, slots.ctypes.data, cow.ctypes.data,
                                    ctypes.byref(ncow)))
        if cow_out is None:
            return slots, cow[:ncow.value].copy()
        return slots[:n], cow[:ncow.value]

    def free(self, seq_id: int):
        _check(lib().pkv_seq_free(self._h, seq_id))

    def stats(self) -> dict:
        """Pool occupancy (pkv_alloc_stats_get) as a dict of the struct's fields."""
        st = _AllocStats()
        _check(lib().pkv_alloc_stats_get(self._h, ctypes.byref(st)))
        return {name: int(getattr(st, name)) for name, _ in _AllocStats._fields_}

    def swap_to(self, other: "BlockAllocator", seq_id: int) -> np.ndarray:
        """Move a sequence into `other` (pkv_seq_swap); returns int32 [n, 2] of (block here,
        block in other) to copy with swap_blocks before the freed blocks are written."""
        _, nb = self.seq_info(seq_id)
        pairs = np.zeros((max(nb, 1), 2), dtype=np.int32)
        n = ctypes.c_int(0)
        _check(lib().pkv_seq_swap(self._h, other._h, seq_id, pairs.ctypes.data, ctypes.byref(n)))
        return pairs[:n.value]

    def block_tables(self, seq_ids, max_blocks: int, tables_out=None, lens_out=None):
        """Block tables [n, max_blocks] (padded with -1) and lengths [n], int32; filled into
        tables_out / lens_out when given (contiguous int32 arrays of those shapes)."""
        ids = _np(seq_ids, np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32) if tables_out is None else tables_out
        lens = np.empty(len(ids), dtype=np.int32) if lens_out is None else lens_out
        if tables.dtype != np.int32 or tables.shape != (len(ids), max_blocks) or not tables.flags.c_contiguous:
            raise ValueError("tables_out must be a contiguous int32 [n, max_blocks] array")
        if lens.dtype != np.int32 or lens.shape != (len(ids),):
            raise ValueError("lens_out must be an int32 [n] array")
        _check(lib().pkv_alloc_block_tables(self._h, ids.ctypes.data, len(ids), max_blocks,
                                            tables.ctypes.data, lens.ctypes.data))
        return tables, lens

    @property
    def num_free(self) -> int:
        return lib().pkv_alloc_num_free(self._h)

    @property
    def num_seqs(self) -> int:
        return lib().pkv_alloc_num_seqs(self._h)

    def prefix_groups(self, seq_ids, max_chunk: int):
        """pkv_alloc_prefix_groups: (chunk_first, chunk_src, group_blocks) int32 [n] host arrays."""
        ids = _np(seq_ids, np.int64)
        n = len(ids)
        first, src, blocks = (np.zeros(n, np.int32) for _ in range(3))
        _check(lib().pkv_alloc_prefix_groups(self._h, ids.ctypes.data, n, int(max_chunk), first.ctypes.data,
                                             src.ctypes.data, blocks.ctypes.data))
        return first, src, blocks

    def shared_prefix_blocks(self, seq_ids) -> np.ndarray:
        """Leading blocks of each sequence with a reference count above 1, int32 [n]
        (pkv_alloc_shared_prefix_blocks): the attention calls' shared_prefix_blocks hint."""
        ids = _np(seq_ids, np.int64)
        out = np.empty(len(ids), dtype=np.int32)
        _check(lib().pkv_alloc_shared_prefix_blocks(self._h, ids.ctypes.data, len(ids), out.ctypes.data))
        return out

    def refcount(self, block: int) -> int:
        return lib().pkv_alloc_refcount(self._h, block)

    def seq_info(self, seq_id: int):
        length = ctypes.c_int64(0)
        nb = ctypes.c_int(0)
        _check(lib().pkv_seq_info(self._h, seq_id, ctypes.byref(length), ctypes.byref(nb)))
        return length.value, nb.value

    def free_list(self) -> np.ndarray:
        n = lib().pkv_alloc_free_list(self._h, None, 0)
        out = np.empty(n, dtype=np.int32)
        lib().pkv_alloc_free_list(self._h, out.ctypes.data, n)
        return out
