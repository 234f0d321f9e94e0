"""A paged KV cache on one device: the host block pool plus the two device pools.

Host bookkeeping (which block, which slot) is the C++ pool behind ``binding.BlockPool``;
every byte written into the device pools goes through the library: rows through
``pkv_kv_cache_append``, copy-on-write block copies through ``pkv_copy_blocks``.  torch only
provides the device memory.
"""

from __future__ import annotations

import numpy as np

from . import binding

_PREFIX_BASE = 1 << 40  # sequence ids used for shared prefixes while building groups


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device,
                 free_order=None, block_size: int = 16, fill=None, pinned: bool = False):
        """``pinned``: the pools live in pinned host memory (device must be "cpu"), e.g. as the
        swap space that ``move_to`` moves sequences into and out of."""
        import torch

        self.pool = binding.BlockPool(num_blocks, block_size, free_order)
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        if pinned and str(device) != "cpu":
            raise ValueError("pinned pools live on the host (device='cpu')")
        mk = dict(dtype=dtype, device=device, pin_memory=pinned)
        if fill is None:
            self.k_cache = torch.empty(shape, **mk)
            self.v_cache = torch.empty(shape, **mk)
        else:
            self.k_cache = torch.full(shape, fill, **mk)
            self.v_cache = torch.full(shape, fill, **mk)
        self.block_size = block_size
        self.device = device
        self.pinned = pinned

    def _device_pools(self, what: str) -> None:
        if self.pinned:
            raise ValueError(f"{what}: a pinned host cache is a swap space; sequences enter it with move_to")

    # -------------------------------------------------------------------- writing
    def write(self, slots, key, value, chunk_tokens: int = 1 << 15) -> None:
        """Scatter rows key/value [T, Hkv, D] to int64 ``slots`` through the append kernel."""
        import torch

        self._device_pools("write")
        slots = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64))
        T = int(slots.numel())
        for a in range(0, T, chunk_tokens):
            b = min(T, a + chunk_tokens)
            sl = slots[a:b].to(self.device)
            k = key[a:b].to(self.device).contiguous()
            v = value[a:b].to(self.device).contiguous()
            binding.kv_cache_append(k, v, self.k_cache, self.v_cache, sl)

    def copy_blocks(self, pairs) -> None:
        """Copy-on-write: duplicate block src into dst in both pools (pkv_copy_blocks, one launch)."""
        import torch

        pairs = list(pairs)
        if not pairs:
            return
        self._device_pools("copy_blocks")
        t = torch.tensor(pairs, dtype=torch.int32).reshape(-1, 2).to(self.device)
        binding.copy_blocks(self.k_cache, self.v_cache, t)

    # ---------------------------------------------------------------- sequences
    def add_sequence(self, seq: int, key, value) -> np.ndarray:
        """New sequence holding key/value [L, Hkv, D]; returns its slots."""
        self.pool.seq_allocate(seq, 0)
        return self.extend(seq, key, value)

    def extend(self, seq: int, key, value) -> np.ndarray:
        slots, cow = self.pool.seq_extend(seq, int(key.shape[0]))
        self.copy_blocks(cow)
        if len(slots):
            self.write(slots, key, value)
        return slots

    def move_to(self, other: "PagedKVCache", seqs) -> np.ndarray:
        """Swap: move whole sequences into ``other`` (device pools <-> pinned host pools).  The
        host pools do the bookkeeping (pkv_pool_move_seqs) and one pkv_swap_blocks launch
        moves the blocks, enqueued before anything can reuse the freed blocks.  Returns the
        (block here, block there) pairs."""
        import torch

        pairs = self.pool.move_seqs(other.pool, seqs)
        if len(pairs):
            gpu = self.device if str(self.device) != "cpu" else other.device
            binding.swap_blocks(other.k_cache, other.v_cache, self.k_cache, self.v_cache,
                                torch.from_numpy(np.ascontiguousarray(pairs)).to(gpu))
        return pairs

    def fork(self, parent: int, child: int) -> None:
        self.pool.seq_fork(parent, child)

    def free(self, seq: int) -> None:
        self.pool.seq_free(seq)

    def append_tokens(self, seqs, key, value) -> np.ndarray:
        """One new token per sequence (key/value [B, Hkv, D]); returns the B slots.

        Host side: each sequence takes its slot (new block when the last one is full,
        copy-on-write when it is shared).  Device side: one append launch for all B rows.
        """
        all_slots = np.zeros(len(seqs), dtype=np.int64)
        for i, s in enumerate(seqs):
            slots, cow = self.pool.seq_extend(int(s), 1)
            self.copy_blocks(cow)
            all_slots[i] = slots[0]
        self.write(all_slots, key, value)
        return all_slots

    def tables(self, seqs, max_blocks_per_seq: int | None = None):
        """Device (block_tables int32 [B, maxb], context_lens int32 [B]) and the max length."""
        import torch

        lens = [self.pool.seq_context_len(int(s)) for s in seqs]
        maxc = max(lens) if lens else 0
        if max_blocks_per_seq is None:
            max_blocks_per_seq = max(1, -(-maxc // self.block_size))
        bt, ctx = self.pool.block_tables(list(seqs), max_blocks_per_seq)
        return (torch.from_numpy(np.ascontiguousarray(bt)).to(self.device),
                torch.from_numpy(np.ascontiguousarray(ctx)).to(self.device), int(maxc))


def build_cache(workload, device, fill=None) -> PagedKVCache:
    """Fill a cache with every sequence of a ``workloads.Workload`` (before its append).

    Prefix groups are built the way shared prefixes arise: the prefix is written once
    under its own id, each member forks it (sharing the blocks, ref + 1), the member's own
    tokens are appended, and the prefix id is released -- leaving every prefix block with
    one reference per member.
    """
    import torch

    sp = workload.spec
    dtype = getattr(torch, sp.dtype)
    cache = PagedKVCache(workload.num_blocks, sp.num_kv_heads, sp.head_dim, dtype, device,
                         free_order=workload.free_order, block_size=sp.block_size, fill=fill)
    if workload.groups is None:
        for s in range(sp.num_seqs):
            k, v = workload.seq_kv(s)
            cache.add_sequence(s, k, v)
    else:
        for gi, members in enumerate(workload.groups):
            pk, pv = workload.prefix_kv(gi)
            pid = _PREFIX_BASE + gi
            cache.add_sequence(pid, pk, pv)
            for s in members:
                cache.fork(pid, s)
                k, v = workload.own_kv(s)
                cache.extend(s, k, v)
            cache.free(pid)
    return cache
