"""Reference for the KV append scatter and for block-table gathers -- test infrastructure only.

Layout.  The gtnt.cn page "vLLM推理加速框架：PagedAttention与连续批处理技术解析" §2.1
gives one block's data the shape (block size, heads, head size) and doubles the per-token
cost for K and V; so each of the two pools is ``[num_blocks, block_size, Hkv, D]``.  The
111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解"
§3.2-§3.3 says a new token is written at the end of the sequence's last block, or into a
freshly taken block when the last one is full, and that the block table maps logical
blocks to physical ones.

A *slot* names one token row of the pool: ``slot = physical_block * block_size + offset``.
Token ``t`` of a sequence with block table ``bt`` lives in physical block ``bt[t //
block_size]`` at offset ``t % block_size``.  A negative slot means "no row" (padding).

Both functions work on raw element arrays and copy rows verbatim, so for any dtype the
result is bit-exact by construction.
"""

from __future__ import annotations

import numpy as np


def kv_cache_append(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray,
                    value: np.ndarray, slot_mapping, block_size: int):
    """Return new (k_cache, v_cache) with each new token's row written to its slot.

    ``k_cache``, ``v_cache``: [NB, block_size, Hkv, D]; ``key``, ``value``: [T, Hkv, D];
    ``slot_mapping``: T integers.  Row ``i`` goes to block ``slot // block_size``, offset
    ``slot % block_size``; slots < 0 are skipped.  Everything else is left as it was.
    Written one token at a time, as the append step on the 111cn.net page §3.3 is.
    """
    new_k = np.array(k_cache, copy=True)
    new_v = np.array(v_cache, copy=True)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(int(slot), block_size)
        new_k[block, offset] = key[i]
        new_v[block, offset] = value[i]
    return new_k, new_v


def gather_sequence(cache: np.ndarray, block_table, context_len: int) -> np.ndarray:
    """Read a sequence's rows back out of a pool in logical order: [context_len, Hkv, D].

    Token ``t`` is read from ``cache[block_table[t // bs], t % bs]`` -- the block-table
    lookup of the yunthe.com page "大模型推理显存优化实战：PagedAttention机制原理与vLLM
    连续批处理配置", section "PagedAttention分页注意力机制原理", written out per token.
    """
    bs = cache.shape[1]
    rows = []
    for t in range(context_len):
        rows.append(cache[int(block_table[t // bs]), t % bs])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)
