"""Seeded synthetic workloads for paged decode attention.

This module only draws inputs: context lengths, the pool's initial free-list order, queries,
per-sequence contiguous K/V and the K/V of the token each decode step appends.  It holds
none of the attention or paging arithmetic, so both the fp64 oracle and the HIP path can be
fed from it.  Random numbers come from numpy's PCG64 through ``SeedSequence.spawn``, one
independent stream per purpose and one per sequence (or per shared prefix), so any single
sequence can be regenerated without drawing the others.

Values are standard normal, drawn in float32 and rounded to the workload dtype with
round-to-nearest-even (torch CPU casts).

The five workloads mirror the shapes the pages talk about (the pages publish no data set
for this path, so these stand in for the serving traffic they describe):

* ``tiny_fp32``     -- 4 sequences of {1, 17, 33, 100} tokens, 4 = 4 heads, D 64, fp32, a
  64-block pool; a correctness case.
* ``mha_fp16``      -- Llama-2-7B-like: batch 64, 32 = 32 heads, D 128, fp16, lengths
  uniform in [128, 2048].
* ``gqa_bf16``      -- Llama-3-70B-like: batch 256 (the pages' max-num-seqs 256), 64 query
  heads on 8 KV heads, D 128, bf16, lengths lognormal (median 512, sigma 1) clipped to
  [16, 8192] (the pages' max_model_len 8192).
* ``long_bf16``     -- batch 8 of 32768 tokens, 32 query / 8 KV heads, D 128, bf16.
* ``prefix_bf16``   -- 16 groups of 8 sequences; each group shares one 1024-token prefix
  (the pages' input length 1024), then every sequence has a private suffix of 1..512
  tokens; 64 query / 8 KV heads, D 128, bf16.
* ``single_long_bf16`` -- one sequence of 32768 tokens, 64 query / 8 KV heads, D 128, bf16
  (batch-1 long-context decode, beside the five above).

Block size is 16 everywhere.  The pool holds 10% more blocks than the workload needs,
counting the block each sequence may take for the appended token (``tiny_fp32`` uses 64).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_SIZE = 16

_DTYPES = ("float32", "float16", "bfloat16")


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    dtype: str              # "float32" | "float16" | "bfloat16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: str            # "fixed" | "uniform" | "lognormal" | "prefix"
    fixed_lengths: tuple = ()
    len_lo: int = 0         # uniform: inclusive range; lognormal: clip range
    len_hi: int = 0
    lognormal_median: float = 512.0
    lognormal_sigma: float = 1.0
    prefix_len: int = 0     # "prefix": shared tokens per group
    group_size: int = 1     # "prefix": sequences per group
    suffix_lo: int = 1
    suffix_hi: int = 1
    num_blocks: int = 0     # 0 -> sized from the lengths (+10%)
    block_size: int = BLOCK_SIZE

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


SPECS = {
    "tiny_fp32": Spec("tiny_fp32", "float32", 4, 4, 4, 64, "fixed",
                      fixed_lengths=(1, 17, 33, 100), num_blocks=64),
    "mha_fp16": Spec("mha_fp16", "float16", 64, 32, 32, 128, "uniform",
                     len_lo=128, len_hi=2048),
    "gqa_bf16": Spec("gqa_bf16", "bfloat16", 256, 64, 8, 128, "lognormal",
                     len_lo=16, len_hi=8192, lognormal_median=512.0, lognormal_sigma=1.0),
    "long_bf16": Spec("long_bf16", "bfloat16", 8, 32, 8, 128, "fixed",
                      fixed_lengths=(32768,) * 8),
    "prefix_bf16": Spec("prefix_bf16", "bfloat16", 128, 64, 8, 128, "prefix",
                        prefix_len=1024, group_size=8, suffix_lo=1, suffix_hi=512),
    # one long sequence at the 70B head shape (batch-1 long-context decode; not one of the
    # five workloads above)
    "single_long_bf16": Spec("single_long_bf16", "bfloat16", 1, 64, 8, 128, "fixed",
                             fixed_lengths=(32767,)),
}

# Stream indices under SeedSequence(seed).spawn(_NUM_STREAMS)
_S_LENGTHS, _S_FREE, _S_Q, _S_NEW, _S_KV, _S_PREFIX = range(6)
_NUM_STREAMS = 6


def _cast(a: np.ndarray, dtype: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(getattr(torch, dtype))


def _blocks(n: int, bs: int) -> int:
    return -(-n // bs)


class Workload:
    """Inputs of one decode step of one layer, drawn from ``seed``."""

    def __init__(self, spec: Spec, seed: int = 0):
        if spec.dtype not in _DTYPES:
            raise ValueError(f"dtype {spec.dtype}")
        self.spec = spec
        self.seed = seed
        ss = np.random.SeedSequence(seed)
        streams = ss.spawn(_NUM_STREAMS)
        self._kv_seeds = streams[_S_KV].spawn(spec.num_seqs)
        bs = spec.block_size

        rng = np.random.default_rng(streams[_S_LENGTHS])
        B = spec.num_seqs
        self.groups = None  # list of lists of sequence indices sharing one prefix
        if spec.lengths == "fixed":
            if len(spec.fixed_lengths) != B:
                raise ValueError("fixed_lengths must have num_seqs entries")
            lens = np.array(spec.fixed_lengths, dtype=np.int64)
        elif spec.lengths == "uniform":
            lens = rng.integers(spec.len_lo, spec.len_hi, size=B, endpoint=True)
        elif spec.lengths == "lognormal":
            z = rng.standard_normal(B)
            lens = np.clip(np.round(spec.lognormal_median * np.exp(spec.lognormal_sigma * z)),
                           spec.len_lo, spec.len_hi).astype(np.int64)
        elif spec.lengths == "prefix":
            if B % spec.group_size:
                raise ValueError("num_seqs must be a multiple of group_size")
            suf = rng.integers(spec.suffix_lo, spec.suffix_hi, size=B, endpoint=True)
            lens = spec.prefix_len + suf
            self.groups = [list(range(g * spec.group_size, (g + 1) * spec.group_size))
                           for g in range(B // spec.group_size)]
            self._prefix_seeds = streams[_S_PREFIX].spawn(len(self.groups))
        else:
            raise ValueError(spec.lengths)
        self.context_lens = lens.astype(np.int32)

        # Pool size: blocks for every token incl. the appended one, shared prefixes once.
        if spec.num_blocks:
            nb = spec.num_blocks
        else:
            need = sum(_blocks(int(L) + 1, bs) for L in self.context_lens)
            if self.groups is not None:
                # whole prefix blocks are shared; a partly filled last prefix block is
                # copied by every member on its first append (copy-on-write)
                shared = spec.prefix_len // bs
                need -= shared * (B - len(self.groups))
                if spec.prefix_len % bs:
                    need += len(self.groups)  # the original partial block, until freed
            nb = int(math.ceil(1.1 * need))
        self.num_blocks = nb
        self.free_order = np.random.default_rng(streams[_S_FREE]).permutation(nb).astype(np.int32)

        Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
        self.q = _cast(np.random.default_rng(streams[_S_Q]).standard_normal((B, Hq, D), dtype=np.float32),
                       spec.dtype)
        rng_new = np.random.default_rng(streams[_S_NEW])
        self.new_k = _cast(rng_new.standard_normal((B, Hkv, D), dtype=np.float32), spec.dtype)
        self.new_v = _cast(rng_new.standard_normal((B, Hkv, D), dtype=np.float32), spec.dtype)

    # ------------------------------------------------------------------------------
    @property
    def scale(self) -> float:
        return self.spec.scale

    def group_of(self, s: int):
        if self.groups is None:
            return None
        return s // self.spec.group_size

    def prefix_kv(self, g: int):
        """Contiguous (K, V) [prefix_len, Hkv, D] of shared prefix ``g``."""
        sp = self.spec
        rng = np.random.default_rng(self._prefix_seeds[g])
        shape = (sp.prefix_len, sp.num_kv_heads, sp.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        return _cast(k, sp.dtype), _cast(v, sp.dtype)

    def own_kv(self, s: int):
        """(K, V) of the tokens sequence ``s`` owns alone (the suffix, for prefix groups)."""
        sp = self.spec
        n = int(self.context_lens[s]) - (sp.prefix_len if self.groups is not None else 0)
        rng = np.random.default_rng(self._kv_seeds[s])
        shape = (n, sp.num_kv_heads, sp.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        return _cast(k, sp.dtype), _cast(v, sp.dtype)

    def seq_kv(self, s: int):
        """Contiguous (K, V) [L_s, Hkv, D] of sequence ``s`` in logical order."""
        k, v = self.own_kv(s)
        if self.groups is None:
            return k, v
        import torch

        pk, pv = self.prefix_kv(self.group_of(s))
        return torch.cat([pk, k]), torch.cat([pv, v])

    def seq_kv_after_append(self, s: int):
        """(K, V) [L_s + 1, Hkv, D]: the sequence followed by its appended token."""
        import torch

        k, v = self.seq_kv(s)
        return torch.cat([k, self.new_k[s:s + 1]]), torch.cat([v, self.new_v[s:s + 1]])

    def kv_bytes(self, with_append: bool = True) -> int:
        """Bytes of K plus V that one decode over every context reads."""
        sp = self.spec
        e = {"float32": 4, "float16": 2, "bfloat16": 2}[sp.dtype]
        tokens = int(self.context_lens.sum()) + (sp.num_seqs if with_append else 0)
        return tokens * sp.num_kv_heads * sp.head_dim * 2 * e


def make_workload(name_or_spec, seed: int = 0, **overrides) -> Workload:
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    if overrides:
        spec = spec.replace(**overrides)
    return Workload(spec, seed)
