"""ctypes binding of libpagedkv (declared in include/pagedkv.h).

Argument marshalling only: tensors become device pointers, shapes become the pool
descriptor, the current torch stream becomes the hipStream_t.  Every computation runs in
the library's HIP kernels; there is no fallback.  If the library is missing, every entry
point raises -- build it with ``__graft_entry__.build()``.

Names mirror the C entry points without the ``pkv_`` prefix.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

OK = 0
STATUS_NAMES = {
    0: "PKV_OK", 1: "PKV_ERR_INVALID_ARGUMENT", 2: "PKV_ERR_UNSUPPORTED",
    3: "PKV_ERR_OUT_OF_BLOCKS", 4: "PKV_ERR_NOT_FOUND", 5: "PKV_ERR_WORKSPACE_TOO_SMALL",
    6: "PKV_ERR_HIP", 7: "PKV_ERR_ALREADY_EXISTS", 8: "PKV_ERR_HOST_MEMORY",
}
DTYPE_CODES = {"float32": 0, "float16": 1, "bfloat16": 2}

# Every symbol include/pagedkv.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_status_string": (ctypes.c_char_p, [_I32]),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_kv_cache_append": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P]),
    "pkv_paged_attn_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attn_partition_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attn_decode": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                     ctypes.c_float, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_paged_attn_decode_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                            _I32, ctypes.c_float, _P, ctypes.c_size_t, _I32, _P]),
    "pkv_copy_blocks": (_I32, [_P, _P, _P, _P, _I32, _P]),
    "pkv_swap_blocks": (_I32, [_P, _P, _I32, _P, _P, _I32, _P, _P, _I32, _P]),
    "pkv_pool_move_seqs": (_I32, [_P, _P, _PI64, _I32, _PI32, _I32, _PI32]),
    "pkv_pool_prefix_groups": (_I32, [_P, _PI64, _I32, _I32, _PI32, _PI32, _PI32, _PI32, _PI32]),
    "pkv_paged_attn_decode_prefix": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, ctypes.c_float,
                                            _P, _P, _P, _I32, _I32, _P, ctypes.c_size_t, _P]),
    "pkv_paged_attn_decode_prefix_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pkv_paged_attn_decode_prefix_append": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                                   ctypes.c_float, _P, _P, _P, _I32, _I32, _P, ctypes.c_size_t, _P]),
    "pkv_set_merge_spin_limit": (_I32, [_I32]),
    "pkv_paged_attn_decode_append_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                                    ctypes.c_float, _I32, _P]),
    "pkv_paged_attn_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "pkv_pool_create": (_I32, [_I32, _I32, _PI32, ctypes.POINTER(_P)]),
    "pkv_pool_destroy": (None, [_P]),
    "pkv_pool_num_blocks": (_I32, [_P]),
    "pkv_pool_block_size": (_I32, [_P]),
    "pkv_pool_num_free": (_I32, [_P]),
    "pkv_pool_ref_count": (_I32, [_P, _I32]),
    "pkv_pool_free_list": (_I32, [_P, _PI32, _I32]),
    "pkv_pool_num_seqs": (_I32, [_P]),
    "pkv_seq_allocate": (_I32, [_P, _I64, _I32, _PI32]),
    "pkv_seq_extend": (_I32, [_P, _I64, _I32, _PI64, _PI32, _PI32]),
    "pkv_seq_fork": (_I32, [_P, _I64, _I64]),
    "pkv_seq_free": (_I32, [_P, _I64]),
    "pkv_seq_context_len": (_I64, [_P, _I64]),
    "pkv_pool_block_tables": (_I32, [_P, _PI64, _I32, _I32, _PI32, _PI32]),
}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))


class OutOfBlocks(PkvError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != OK:
        msg = lib().pkv_last_error().decode(errors="replace")
        cls = OutOfBlocks if status == 3 else PkvError
        raise cls(status, msg or STATUS_NAMES.get(status, str(status)))


def version() -> str:
    return lib().pkv_version().decode()


# ------------------------------------------------------------------------- device
def _dtype_name(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def cache_desc(k_cache) -> CacheDesc:
    """Descriptor of a pool tensor shaped [num_blocks, block_size, num_kv_heads, head_dim]."""
    if k_cache.dim() != 4 or not k_cache.is_contiguous():
        raise ValueError("cache must be a contiguous [num_blocks, block_size, Hkv, D] tensor")
    nb, bs, hkv, d = k_cache.shape
    name = _dtype_name(k_cache)
    if name not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {name}")
    return CacheDesc(nb, bs, hkv, d, DTYPE_CODES[name])


def _same(*ts):
    base = ts[0]
    for t in ts[1:]:
        if t.dtype != base.dtype:
            raise ValueError("tensors must share one dtype")
        if t.device != base.device:
            raise ValueError("tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _on_device(device, *ts):
    """Index arrays the kernels read (tables, lengths, slots, pairs) must live on the launch
    device: a host tensor's pointer would reach the GPU as an address it cannot read."""
    for t in ts:
        if t.device != device:
            raise ValueError(f"a {tuple(t.shape)} tensor is on {t.device}, not on {device}")


def _workspace(nbytes, device, stream):
    """A workspace from torch's caching allocator, allocated on the stream the call is launched
    on, so that the allocator does not hand its memory out again before that stream has run
    the call."""
    import torch

    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    s = torch.cuda.ExternalStream(stream, device=device) if isinstance(stream, int) else stream
    with torch.cuda.stream(s):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kv_cache_append(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """pkv_kv_cache_append: key/value [T, Hkv, D] into the pools at int64 slot_mapping [T]."""
    import torch

    _same(key, value, k_cache, v_cache)
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    desc = cache_desc(k_cache)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    T = key.shape[0]
    if tuple(key.shape) != (T, desc.num_kv_heads, desc.head_dim) or tuple(value.shape) != tuple(key.shape):
        raise ValueError("key/value must be [T, Hkv, D]")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    _on_device(k_cache.device, slot_mapping)
    _check(lib().pkv_kv_cache_append(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                      ctypes.byref(desc), _ptr(slot_mapping), T, _stream(stream)))


def _pairs_arg(pairs):
    import torch

    if pairs.dtype != torch.int32 or not pairs.is_contiguous() or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be a contiguous int32 tensor [n, 2]")
    return int(pairs.shape[0])


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """pkv_copy_blocks: block pairs[i, 0] onto block pairs[i, 1] in both pools (copy-on-write)."""
    _same(k_cache, v_cache)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    n = _pairs_arg(pairs)
    _on_device(k_cache.device, pairs)
    desc = cache_desc(k_cache)
    _check(lib().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(pairs), n, _stream(stream)))


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, stream=None) -> None:
    """pkv_swap_blocks: block pairs[i, 0] of (src_k, src_v) onto block pairs[i, 1] of
    (dst_k, dst_v); either side device memory or pinned host memory."""
    for a in (dst_k, dst_v, src_k, src_v):
        if not a.is_contiguous() or a.dtype != dst_k.dtype or tuple(a.shape[1:]) != tuple(dst_k.shape[1:]):
            raise ValueError("pools must be contiguous with one block shape and dtype")
    if tuple(dst_v.shape) != tuple(dst_k.shape) or tuple(src_v.shape) != tuple(src_k.shape):
        raise ValueError("K and V pools of one side differ in shape")
    n = _pairs_arg(pairs)
    desc = cache_desc(dst_k)
    _check(lib().pkv_swap_blocks(_ptr(dst_k), _ptr(dst_v), int(dst_k.shape[0]), _ptr(src_k), _ptr(src_v),
                                 int(src_k.shape[0]), ctypes.byref(desc), _ptr(pairs), n, _stream(stream)))


def _dtype_code(dtype) -> int:
    """pkv_dtype code of a dtype given as a code, a name ("bfloat16") or a torch dtype."""
    if isinstance(dtype, int):
        return dtype
    name = dtype if isinstance(dtype, str) else str(dtype).replace("torch.", "")
    if name not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {name}")
    return DTYPE_CODES[name]


def paged_attn_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                               partition_size=0, dtype="bfloat16") -> int:
    return int(lib().pkv_paged_attn_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                    max_context_len, partition_size, _dtype_code(dtype)))


def paged_attn_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size=0, dtype="bfloat16") -> int:
    return int(lib().pkv_paged_attn_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                   max_context_len, partition_size, _dtype_code(dtype)))


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                      scale, workspace=None, partition_size=0, stream=None) -> None:
    """pkv_paged_attn_decode.  ``workspace``: a uint8/float device tensor or None (then a
    torch buffer of the needed size is taken from the caching allocator)."""
    import torch

    _same(out, q, k_cache, v_cache)
    desc = cache_desc(k_cache)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or D != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, D] with the cache's D")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if not block_tables.is_contiguous() or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be contiguous [B, max_blocks_per_seq]")
    if context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous [B]")
    _on_device(q.device, block_tables, context_lens)
    need = paged_attn_workspace_bytes(B, Hq, desc.num_kv_heads, D, max_context_len, partition_size, desc.dtype)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), int(max_context_len),
        B, Hq, float(scale), _ptr(workspace), ws_bytes, int(partition_size), _stream(stream)))


def set_merge_spin_limit(limit: int) -> int:
    """pkv_set_merge_spin_limit (a test hook): polls after which the merge launch's bounded
    waits give up; a negative value restores the default.  Returns the previous limit."""
    return int(lib().pkv_set_merge_spin_limit(int(limit)))


def workspace_status(workspace) -> int:
    """The status word at the start of an even-split workspace (a device tensor), read after
    the stream has finished the call: 0, or 1 if a bounded wait of the merge launch gave up."""
    import torch

    return int(workspace.reshape(-1).view(torch.uint8)[:4].view(torch.int32).cpu().item())


def paged_attn_decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                             max_prefix_tokens, dtype="bfloat16") -> int:
    return int(lib().pkv_paged_attn_decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                                  max_context_len, max_prefix_tokens,
                                                                  _dtype_code(dtype)))


def paged_attn_decode_prefix(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                             seq_prefix, group_offsets, group_members, max_prefix_tokens, workspace=None,
                             stream=None) -> None:
    """pkv_paged_attn_decode_prefix: decode with each group's shared prefix read once per group.
    seq_prefix / group_offsets / group_members: int32 device tensors (pkv_pool_prefix_groups)."""
    import torch

    _same(out, q, k_cache, v_cache)
    desc = cache_desc(k_cache)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or D != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, D] with the cache's D")
    for t in (block_tables, context_lens, seq_prefix, group_offsets, group_members):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("tables, lengths and group arrays must be contiguous int32")
    if seq_prefix.numel() != B or group_offsets.numel() < 1:
        raise ValueError("seq_prefix must have B entries, group_offsets at least one")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks_per_seq] and context_lens [B]")
    _on_device(q.device, block_tables, context_lens, seq_prefix, group_offsets, group_members)
    ng = group_offsets.numel() - 1
    need = paged_attn_decode_prefix_workspace_bytes(B, Hq, desc.num_kv_heads, D, max_context_len, max_prefix_tokens,
                                                    desc.dtype)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), int(max_context_len), B, Hq, float(scale), _ptr(seq_prefix),
        _ptr(group_offsets), _ptr(group_members), ng, int(max_prefix_tokens), _ptr(workspace), ws_bytes,
        _stream(stream)))


def paged_attn_decode_prefix_append(out, q, new_key, new_value, k_cache, v_cache, block_tables, context_lens,
                                    max_context_len, scale, seq_prefix, group_offsets, group_members,
                                    max_prefix_tokens, workspace=None, stream=None) -> None:
    """pkv_paged_attn_decode_prefix_append: append new_key/new_value [B, Hkv, D] as each
    sequence's last token, then decode with each group's shared prefix read once per group.
    The group arrays as for paged_attn_decode_prefix (from the extended tables)."""
    import torch

    _same(out, q, k_cache, v_cache, new_key, new_value)
    desc = cache_desc(k_cache)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or D != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, D] with the cache's D")
    if tuple(new_key.shape) != (B, desc.num_kv_heads, D) or tuple(new_value.shape) != tuple(new_key.shape):
        raise ValueError("new_key/new_value must be [B, Hkv, D]")
    for t in (block_tables, context_lens, seq_prefix, group_offsets, group_members):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("tables, lengths and group arrays must be contiguous int32")
    if seq_prefix.numel() != B or group_offsets.numel() < 1:
        raise ValueError("seq_prefix must have B entries, group_offsets at least one")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks_per_seq] and context_lens [B]")
    _on_device(q.device, block_tables, context_lens, seq_prefix, group_offsets, group_members)
    ng = group_offsets.numel() - 1
    need = paged_attn_decode_prefix_workspace_bytes(B, Hq, desc.num_kv_heads, D, max_context_len, max_prefix_tokens,
                                                    desc.dtype)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_prefix_append(
        _ptr(out), _ptr(q), _ptr(new_key), _ptr(new_value), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc),
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), int(max_context_len), B, Hq, float(scale),
        _ptr(seq_prefix), _ptr(group_offsets), _ptr(group_members), ng, int(max_prefix_tokens), _ptr(workspace),
        ws_bytes, _stream(stream)))


def paged_attn_decode_append(out, q, new_key, new_value, k_cache, v_cache, block_tables,
                             context_lens, max_context_len, scale, workspace=None, partition_size=0,
                             stream=None) -> None:
    """pkv_paged_attn_decode_append: append new_key/new_value [B, Hkv, D] as each sequence's
    last token (the slot its block table gives), then decode.  ``workspace`` as for
    paged_attn_decode."""
    import torch

    _same(out, q, k_cache, v_cache, new_key, new_value)
    desc = cache_desc(k_cache)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or D != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, D] with the cache's D")
    if tuple(new_key.shape) != (B, desc.num_kv_heads, D) or tuple(new_value.shape) != tuple(new_key.shape):
        raise ValueError("new_key/new_value must be [B, Hkv, D]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if not block_tables.is_contiguous() or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be contiguous [B, max_blocks_per_seq]")
    if context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous [B]")
    _on_device(q.device, block_tables, context_lens)
    need = paged_attn_workspace_bytes(B, Hq, desc.num_kv_heads, D, max_context_len, partition_size, desc.dtype)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_append(
        _ptr(out), _ptr(q), _ptr(new_key), _ptr(new_value), _ptr(k_cache), _ptr(v_cache),
        ctypes.byref(desc), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), B, Hq, float(scale), _ptr(workspace), ws_bytes, int(partition_size),
        _stream(stream)))


def paged_attn_decode_append_noalloc(out, q, new_key, new_value, k_cache, v_cache, block_tables,
                                     context_lens, max_context_len, scale, partition_size=0, stream=None) -> None:
    """pkv_paged_attn_decode_append_noalloc: the same step as paged_attn_decode_append with the
    library's per-GPU scratch array as workspace; nothing is allocated (here or in the library)."""
    import torch

    _same(out, q, k_cache, v_cache, new_key, new_value)
    desc = cache_desc(k_cache)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or D != desc.head_dim:
        raise ValueError("q/out must be [B, Hq, D] with the cache's D")
    if tuple(new_key.shape) != (B, desc.num_kv_heads, D) or tuple(new_value.shape) != tuple(new_key.shape):
        raise ValueError("new_key/new_value must be [B, Hkv, D]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if not block_tables.is_contiguous() or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be contiguous [B, max_blocks_per_seq]")
    if context_lens.numel() != B or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous [B]")
    _on_device(q.device, block_tables, context_lens)
    _check(lib().pkv_paged_attn_decode_append_noalloc(
        _ptr(out), _ptr(q), _ptr(new_key), _ptr(new_value), _ptr(k_cache), _ptr(v_cache),
        ctypes.byref(desc), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), B, Hq, float(scale), int(partition_size), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    """pkv_paged_attn_noalloc_scratch_bytes: the per-GPU scratch array's size."""
    return int(lib().pkv_paged_attn_noalloc_scratch_bytes())


# --------------------------------------------------------------------------- host
class BlockPool:
    """Host block pool (pkv_pool_* / pkv_seq_*): free list, ref counts, block tables."""

    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        handle = ctypes.c_void_p()
        if free_order is None:
            _check(lib().pkv_pool_create(num_blocks, block_size, None, ctypes.byref(handle)))
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if fo.size != num_blocks:
                raise ValueError("free_order must have num_blocks entries")
            _check(lib().pkv_pool_create(num_blocks, block_size,
                                         fo.ctypes.data_as(_PI32), ctypes.byref(handle)))
        self._h = handle

    def close(self):
        if self._h:
            lib().pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return lib().pkv_pool_num_blocks(self._h)

    @property
    def block_size(self) -> int:
        return lib().pkv_pool_block_size(self._h)

    def num_free(self) -> int:
        return lib().pkv_pool_num_free(self._h)

    def num_seqs(self) -> int:
        return lib().pkv_pool_num_seqs(self._h)

    def ref_count(self, block_id: int) -> int:
        return lib().pkv_pool_ref_count(self._h, block_id)

    def free_list(self) -> list:
        n = lib().pkv_pool_free_list(self._h, None, 0)
        buf = np.zeros(max(n, 1), dtype=np.int32)
        lib().pkv_pool_free_list(self._h, buf.ctypes.data_as(_PI32), n)
        return buf[:n].tolist()

    def seq_allocate(self, seq: int, num_tokens: int) -> list:
        nb = -(-num_tokens // max(self.block_size, 1)) if num_tokens > 0 else 0
        buf = np.zeros(max(nb, 1), dtype=np.int32)
        _check(lib().pkv_seq_allocate(self._h, seq, num_tokens, buf.ctypes.data_as(_PI32)))
        return buf[:nb].tolist()

    def seq_extend(self, seq: int, n: int):
        """Returns (slots int64 ndarray [n], cow list of (src, dst))."""
        slots = np.zeros(max(n, 1), dtype=np.int64)
        cow = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(lib().pkv_seq_extend(self._h, seq, n, slots.ctypes.data_as(_PI64),
                                    cow.ctypes.data_as(_PI32), ctypes.byref(ncow)))
        return slots[:n], ([(int(cow[0]), int(cow[1]))] if ncow.value else [])

    def seq_fork(self, parent: int, child: int) -> None:
        _check(lib().pkv_seq_fork(self._h, parent, child))

    def seq_free(self, seq: int) -> None:
        _check(lib().pkv_seq_free(self._h, seq))

    def move_seqs(self, dst: "BlockPool", seqs) -> np.ndarray:
        """pkv_pool_move_seqs: move ``seqs`` into pool ``dst``; returns the (src block, dst
        block) pairs to copy, int32 [k, 2]."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        cap = sum(-(-max(self.seq_context_len(int(x)), 0) // self.block_size) for x in s.tolist())
        pairs = np.zeros((max(cap, 1), 2), dtype=np.int32)
        npairs = ctypes.c_int32(0)
        _check(lib().pkv_pool_move_seqs(self._h, dst._h, s.ctypes.data_as(_PI64), s.size,
                                        pairs.ctypes.data_as(_PI32), cap, ctypes.byref(npairs)))
        return pairs[:npairs.value]

    def prefix_groups(self, seqs, min_prefix_tokens: int = 0):
        """pkv_pool_prefix_groups: (seq_prefix int32 [n], group_offsets int32 [g+1],
        group_members int32 [m], max_prefix) for the batch ``seqs``."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.size
        sp = np.zeros(max(n, 1), dtype=np.int32)
        offs = np.zeros(n + 1, dtype=np.int32)
        mem = np.zeros(max(n, 1), dtype=np.int32)
        ng, mx = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().pkv_pool_prefix_groups(self._h, s.ctypes.data_as(_PI64), n, min_prefix_tokens,
                                            sp.ctypes.data_as(_PI32), offs.ctypes.data_as(_PI32),
                                            mem.ctypes.data_as(_PI32), ctypes.byref(ng), ctypes.byref(mx)))
        return sp[:n], offs[:ng.value + 1], mem[:offs[ng.value]], int(mx.value)

    def seq_context_len(self, seq: int) -> int:
        return int(lib().pkv_seq_context_len(self._h, seq))

    def block_tables(self, seqs, max_blocks_per_seq: int):
        """Returns (tables int32 [n, max_blocks_per_seq] padded -1, context_lens int32 [n])."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        n = s.size
        tables = np.zeros((max(n, 1), max(max_blocks_per_seq, 1)), dtype=np.int32)
        lens = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().pkv_pool_block_tables(self._h, s.ctypes.data_as(_PI64), n, max_blocks_per_seq,
                                           tables.ctypes.data_as(_PI32), lens.ctypes.data_as(_PI32)))
        return tables[:n, :max_blocks_per_seq], lens[:n]
