"""Plain, slow, obviously correct CPU oracle for paged decode attention and KV append.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP library
(no kernels, headers, helpers, tables or pre/post-processing) and imports nothing from
``paged_kv_cache_376_amd``.

The pages it follows (cited by title and section throughout):

* "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解" (111cn.net)
  -- block manager sketch in §3.3, paging scheme in §3.2.
* "vLLM推理加速框架：PagedAttention与连续批处理技术解析" (gtnt.cn)
  -- per-block data layout and ref count in §2.1, copy-on-write in §2.2.
* "大模型推理显存优化实战：PagedAttention机制原理与vLLM连续批处理配置" (yunthe.com)
  -- section "PagedAttention分页注意力机制原理": the kernel resolves physical blocks
  through the block table and computes attention over them; blocks are returned to the
  pool when a request ends.

Modules:

* ``attention``     -- fp64 single-query attention over contiguous, un-paged K/V.
* ``kv_append``     -- the append scatter and the block-table gather, written from the
                       layout definition.
* ``block_manager`` -- a pure-Python model of the block pool / block tables.
* ``block_copy``    -- whole-block copies: copy-on-write inside a pool, swap between pools.

Every function here is pinned by ``tests/test_oracle_*.py`` against brute force, closed
forms, an independent library routine and hand-worked fixtures in ``tests/golden/``.
"""

from .attention import decode_attention, decode_attention_single
from .kv_append import kv_cache_append, gather_sequence
from .block_manager import BlockManager, OutOfBlocks
from .block_copy import copy_blocks, swap_blocks

__all__ = [
    "decode_attention",
    "decode_attention_single",
    "kv_cache_append",
    "gather_sequence",
    "BlockManager",
    "OutOfBlocks",
    "copy_blocks",
    "swap_blocks",
]
