"""The benchmark's byte accounting (CPU): algorithmic bytes of the plain decode and of the
prefix-shared decode, counted by hand on small workloads."""

import numpy as np

import bench
from paged_kv_cache_376_amd import workloads as W


def test_plain_decode_bytes():
    w = W.make_workload("tiny_fp32", 0)  # lengths 1, 17, 33, 100; 4 = 4 heads, D 64, fp32
    kv, dec = bench.algorithmic_bytes(w)
    lens = [2, 18, 34, 101]  # one appended token each
    assert kv == sum(lens) * 4 * 64 * 2 * 4
    assert dec == kv + 2 * 4 * 4 * 64 * 4 + 4 * (1 + 2 + 3 + 7) + 4 * 4


def test_prefix_shared_bytes_count_each_prefix_once():
    spec = W.SPECS["prefix_bf16"].replace(num_seqs=12, group_size=4, prefix_len=320, suffix_hi=40)
    w = W.Workload(spec, seed=5)
    lens = [int(L) + 1 for L in w.context_lens]
    # three groups of four sharing 320 tokens; sequence 7 is left out of every group
    seq_prefix = np.array([320] * 7 + [0] + [320] * 4, dtype=np.int32)
    offs = np.array([0, 4, 7, 11], dtype=np.int32)
    members = np.array([0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 11], dtype=np.int32)
    kv, dec = bench.prefix_shared_bytes(w, seq_prefix, offs, members)
    tokens = 3 * 320 + sum(lens) - 11 * 320
    row = spec.num_kv_heads * spec.head_dim * 2 * 2
    assert kv == tokens * row
    plain_kv, plain_dec = bench.algorithmic_bytes(w)
    assert plain_kv - kv == 8 * 320 * row  # 11 members read the prefix, 3 reads remain
    assert plain_dec - dec == plain_kv - kv


def test_append_bytes_are_counted_once():
    """The fused call reads each new row as part of its context (already in the K/V bytes) and
    writes it once; the append as a call of its own reads and writes the rows and reads the
    8-byte slots."""
    w = W.make_workload("tiny_fp32", 0)
    row = 4 * 64 * 4  # Hkv x D x fp32
    assert bench.fused_append_bytes(w) == 4 * 2 * row  # 4 sequences, K and V written
    assert bench.append_call_bytes(w) == 4 * 2 * row * 2 + 8 * 4
