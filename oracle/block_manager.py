"""Pure-Python model of the block pool and block tables -- test infrastructure only.

Written from the pages' description, not from any implementation:

* 111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解"
  §3.2: the KV cache is cut into fixed blocks of 16 tokens; the GPU memory is a pool of
  equal physical blocks that need not be contiguous; a block table maps the logical order;
  a new physical block is taken only when the current one is full; one physical block may
  be shared by several requests.
  §3.3 (block manager sketch): ``allocate`` takes ceil(num_tokens / block_size) blocks,
  each one popped from the END of the free list; ``append_token`` pops a new block if the
  last block of the sequence is full, otherwise writes at the end of the last block.
  §2.2 (the scheduler): admission checks that the blocks a request needs do not exceed the
  free blocks -- read here as: an operation that would run out of blocks changes nothing.
* gtnt.cn page "vLLM推理加速框架：PagedAttention与连续批处理技术解析" §2.1: every block
  carries a reference count; §2.2: candidates that share a prefix share its blocks and are
  copied on write.
* yunthe.com page "大模型推理显存优化实战：PagedAttention机制原理与vLLM连续批处理配置",
  section "PagedAttention分页注意力机制原理": sequences share prefix KV by referencing the
  same physical blocks; a request's blocks go back to the free pool when it ends.

Readings where the pages are silent (stated again in the design notes):

* "last block full" means the sequence holds a multiple of ``block_size`` tokens (a
  sequence with no tokens has no last block, so its first token also takes a new block);
* appending into a last block that is shared (ref > 1) and not full first copies it into a
  fresh block (copy-on-write); the (source, destination) pair is reported so the caller can
  copy the device bytes.  A full shared last block needs no copy: the token goes to a new
  block anyway;
* ``free`` walks the table in logical order, decrements each block's count and pushes the
  block onto the end of the free list when the count reaches zero;
* ``fork`` gives the child the parent's table and token count and increments every
  block's count;
* a slot is ``physical_block * block_size + offset``;
* a swap moves whole sequences between two pools (``move_seqs``).
"""

from __future__ import annotations


class OutOfBlocks(Exception):
    """The free list cannot cover the request; the pool was left unchanged."""


class SharedWithStayingSequence(Exception):
    """A block of a moving sequence is also used by one that stays; nothing changed."""


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if free_order is None:
            free_order = range(num_blocks)
        self.free_blocks = [int(b) for b in free_order]
        if sorted(self.free_blocks) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.ref_count = [0] * num_blocks
        self.block_tables: dict[int, list[int]] = {}
        self.num_tokens: dict[int, int] = {}

    # -- queries ---------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free_blocks)

    def block_table(self, seq: int) -> list[int]:
        return list(self.block_tables[seq])

    def context_len(self, seq: int) -> int:
        return self.num_tokens[seq]

    # -- operations ------------------------------------------------------------------
    def allocate(self, seq: int, num_tokens: int) -> list[int]:
        """New sequence holding ``num_tokens`` tokens: ceil(n / bs) blocks popped from the end."""
        if seq in self.block_tables:
            raise KeyError(f"sequence {seq} already exists")
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        need = _ceil_div(num_tokens, self.block_size)
        if need > len(self.free_blocks):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free_blocks)} free")
        blocks = [self.free_blocks.pop() for _ in range(need)]
        for b in blocks:
            self.ref_count[b] = 1
        self.block_tables[seq] = blocks
        self.num_tokens[seq] = num_tokens
        return list(blocks)

    def _blocks_needed_for_extend(self, seq: int, n: int) -> int:
        tokens = self.num_tokens[seq]
        table = self.block_tables[seq]
        need = _ceil_div(tokens + n, self.block_size) - _ceil_div(tokens, self.block_size)
        if n > 0 and tokens % self.block_size != 0 and self.ref_count[table[-1]] > 1:
            need += 1  # copy-on-write of a shared, partly filled last block
        return need

    def append_token(self, seq: int):
        """Append one token; returns (slot, cow) where cow is None or (src, dst)."""
        if self._blocks_needed_for_extend(seq, 1) > len(self.free_blocks):
            raise OutOfBlocks("no free block for the next token")
        table = self.block_tables[seq]
        tokens = self.num_tokens[seq]
        offset = tokens % self.block_size
        cow = None
        if offset == 0:
            # last block full (or no block yet): take a fresh one
            new = self.free_blocks.pop()
            self.ref_count[new] = 1
            table.append(new)
        elif self.ref_count[table[-1]] > 1:
            # shared, partly filled last block: copy it before writing
            src = table[-1]
            dst = self.free_blocks.pop()
            self.ref_count[src] -= 1
            self.ref_count[dst] = 1
            table[-1] = dst
            cow = (src, dst)
        self.num_tokens[seq] = tokens + 1
        return table[-1] * self.block_size + offset, cow

    def extend(self, seq: int, n: int):
        """Append ``n`` tokens, all or nothing; returns (slots, cow_pairs)."""
        if seq not in self.block_tables:
            raise KeyError(f"unknown sequence {seq}")
        if n < 0:
            raise ValueError("n must be >= 0")
        if self._blocks_needed_for_extend(seq, n) > len(self.free_blocks):
            raise OutOfBlocks("not enough free blocks for the extension")
        slots, cows = [], []
        for _ in range(n):
            slot, cow = self.append_token(seq)
            slots.append(slot)
            if cow is not None:
                cows.append(cow)
        return slots, cows

    def fork(self, parent: int, child: int) -> None:
        """Child shares every block of the parent (ref + 1 each)."""
        if parent not in self.block_tables:
            raise KeyError(f"unknown sequence {parent}")
        if child in self.block_tables:
            raise KeyError(f"sequence {child} already exists")
        table = list(self.block_tables[parent])
        for b in table:
            self.ref_count[b] += 1
        self.block_tables[child] = table
        self.num_tokens[child] = self.num_tokens[parent]

    def free(self, seq: int) -> None:
        """Drop the sequence; blocks whose count reaches zero return to the free list."""
        if seq not in self.block_tables:
            raise KeyError(f"unknown sequence {seq}")
        for b in self.block_tables.pop(seq):
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                self.free_blocks.append(b)
        del self.num_tokens[seq]

    def move_seqs(self, dst: "BlockManager", seqs):
        """Move sequences into another pool (swap out to host, or back in); returns the
        (block here, block in dst) pairs whose data must be copied.

        The yunthe.com page, section "生产部署注意事项", describes the swap space: when device
        memory runs short some requests' KV cache is moved to host memory and brought back
        later.  Read here as whole sequences changing pools, with these steps:

        1. every listed sequence must exist here and not in ``dst``, and be listed once
           (checked in list order, the first failure reported);
        2. the distinct blocks of their tables are numbered in order of first use (sequences
           in the given order, each table in logical order); each must be referenced only by
           the moving sequences (a block shared with a sequence that stays cannot move);
        3. ``dst`` must have a free block for each of them, else nothing changes;
        4. each such block takes a block popped from the end of ``dst``'s free list, which
           keeps its reference count; the moved tables are rewritten through this map;
        5. the sequences then leave this pool exactly as ``free`` would take them out.
        """
        seqs = [int(x) for x in seqs]
        if dst is self or dst.block_size != self.block_size:
            raise ValueError("destination must be another pool with the same block size")
        for i, s in enumerate(seqs):  # checked in list order
            if s not in self.block_tables:
                raise KeyError(f"unknown sequence {s}")
            if s in dst.block_tables:
                raise KeyError(f"sequence {s} already exists in the destination")
            if s in seqs[:i]:
                raise ValueError(f"sequence {s} is listed twice")
        first_use, count = [], {}
        for s in seqs:
            for b in self.block_tables[s]:
                if b not in count:
                    first_use.append(b)
                    count[b] = 0
                count[b] += 1
        for b in first_use:
            if self.ref_count[b] != count[b]:
                raise SharedWithStayingSequence(f"block {b} is also used by a sequence that stays")
        if len(first_use) > len(dst.free_blocks):
            raise OutOfBlocks(f"need {len(first_use)} blocks, {len(dst.free_blocks)} free")
        new_id = {}
        for b in first_use:
            nb = dst.free_blocks.pop()
            dst.ref_count[nb] = self.ref_count[b]
            new_id[b] = nb
        for s in seqs:
            dst.block_tables[s] = [new_id[b] for b in self.block_tables[s]]
            dst.num_tokens[s] = self.num_tokens[s]
            self.free(s)
        return [(b, new_id[b]) for b in first_use]

    def prefix_groups(self, seqs, min_prefix_tokens: int = 0):
        """Groups of batch entries whose contexts start with the same physical blocks.

        Prefix sharing is sharing by reference: sequences point at the same physical blocks
        for their common start (yunthe.com page, section "PagedAttention分页注意力机制原理";
        111cn.net page §3.2, one physical block shared by several requests).  A shared prefix
        is read off the tables as follows:

        1. batch entries with at least one full block are bucketed by their first block id;
        2. in a bucket of two or more, the prefix is the run of leading table entries equal for
           every member, counting only blocks every member fills completely;
        3. its length in tokens is rounded down to a multiple of 16 (whole 16-token tiles);
        4. a bucket whose prefix is below max(16, min_prefix_tokens) is not a group.

        Returns (seq_prefix per entry, groups as lists of batch positions in batch order, the
        groups ordered by their first member)."""
        seqs = [int(x) for x in seqs]
        bs = self.block_size
        seq_prefix = [0] * len(seqs)
        buckets: dict[int, list[int]] = {}
        for i, s in enumerate(seqs):
            if self.num_tokens[s] // bs >= 1:
                buckets.setdefault(self.block_tables[s][0], []).append(i)
        groups = []
        for members in buckets.values():  # insertion order = order of first appearance
            if len(members) < 2:
                continue
            tabs = [self.block_tables[seqs[i]] for i in members]
            full = min(self.num_tokens[seqs[i]] // bs for i in members)
            k = 0
            while k < full and all(t[k] == tabs[0][k] for t in tabs):
                k += 1
            tokens = (k * bs) // 16 * 16
            if tokens < max(16, min_prefix_tokens):
                continue
            for i in members:
                seq_prefix[i] = tokens
            groups.append(list(members))
        return seq_prefix, groups

    def tables(self, seqs, max_blocks_per_seq: int):
        """Padded table rows (pad -1) and context lengths for ``seqs``, in that order."""
        rows, lens = [], []
        for s in seqs:
            t = self.block_tables[s]
            if len(t) > max_blocks_per_seq:
                raise ValueError("table longer than max_blocks_per_seq")
            rows.append(t + [-1] * (max_blocks_per_seq - len(t)))
            lens.append(self.num_tokens[s])
        return rows, lens
