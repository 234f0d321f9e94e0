"""Reference for whole-block copies: copy-on-write and swap -- test infrastructure only.

Copy-on-write: the gtnt.cn page "vLLM推理加速框架：PagedAttention与连续批处理技术解析"
§2.2 lists copy-on-write among the benefits of paging (candidates of a beam search share the
blocks of their common prefix), and §2.1 gives every block a reference count.  A candidate
that is about to write into a shared block first gets a private copy of it; which blocks is
decided by the block manager (``block_manager.BlockManager.extend`` reports (source,
destination) pairs), and this module moves the data.

Swap: the yunthe.com page "大模型推理显存优化实战：PagedAttention机制原理与vLLM连续批处理配置",
section "生产部署注意事项", describes the swap space: when device memory runs short some
requests' KV cache is moved out to host memory and brought back later.  Read here as whole
blocks moving between a device pool and a host pool of the same block shape.

A block of a pool ``[num_blocks, block_size, Hkv, D]`` is ``pool[b]``.  Both functions copy
blocks verbatim (element arrays, any dtype), so results are bit-exact by construction.  All
pairs of one call read the pools as they were before the call.
"""

from __future__ import annotations

import numpy as np


def _valid(src: int, dst: int, src_blocks: int, dst_blocks: int) -> bool:
    return 0 <= src < src_blocks and 0 <= dst < dst_blocks


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs):
    """Return new (k_pool, v_pool) where, for each (src, dst) in ``pairs``, block ``dst`` holds
    block ``src``'s data.  Pairs naming a block outside the pool, or src == dst, change
    nothing.  Every other block keeps its data."""
    new_k = np.array(k_pool, copy=True)
    new_v = np.array(v_pool, copy=True)
    nb = k_pool.shape[0]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not _valid(src, dst, nb, nb) or src == dst:
            continue
        new_k[dst] = k_pool[src]
        new_v[dst] = v_pool[src]
    return new_k, new_v


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray, pairs):
    """Return new (dst_k, dst_v) where, for each (src, dst) in ``pairs``, block ``dst`` of the
    destination pools holds block ``src`` of the source pools.  Pairs naming a block outside
    its pool change nothing; the source pools are not modified."""
    new_k = np.array(dst_k, copy=True)
    new_v = np.array(dst_v, copy=True)
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not _valid(src, dst, src_k.shape[0], dst_k.shape[0]):
            continue
        new_k[dst] = src_k[src]
        new_v[dst] = src_v[src]
    return new_k, new_v
