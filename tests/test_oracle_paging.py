"""CPU pins of the paging side of the oracle: append scatter, table gather, block manager."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.block_manager import BlockManager, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ------------------------------------------------------------------ append / gather
def test_append_matches_hand_worked_fixture():
    fx = _load("kv_append_worked.json")
    kc = np.array(fx["k_cache"], dtype=np.float32)
    vc = np.array(fx["v_cache"], dtype=np.float32)
    nk, nv = oracle.kv_cache_append(kc, vc, np.array(fx["key"], dtype=np.float32),
                                    np.array(fx["value"], dtype=np.float32),
                                    fx["slot_mapping"], fx["block_size"])
    assert np.array_equal(nk, np.array(fx["expected_k_cache"], dtype=np.float32))
    assert np.array_equal(nv, np.array(fx["expected_v_cache"], dtype=np.float32))
    # inputs untouched (the oracle returns copies)
    assert np.array_equal(kc, np.array(fx["k_cache"], dtype=np.float32))
    g = fx["gather"]
    got = oracle.gather_sequence(nk, g["block_table"], g["context_len"])
    assert np.array_equal(got, np.array(g["expected_k"], dtype=np.float32))


def test_append_then_gather_round_trip_bitwise():
    # tokens appended at the slots a block table implies read back identically, for the
    # raw 16-bit patterns of bf16 as well
    rng = np.random.default_rng(5)
    NB, bs, H, D = 12, 4, 3, 5
    table = rng.permutation(NB)[:4]
    L = 14
    slots = [int(table[t // bs]) * bs + t % bs for t in range(L)]
    kc = rng.integers(0, 2 ** 16, size=(NB, bs, H, D), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(NB, bs, H, D), dtype=np.uint16)
    key = rng.integers(0, 2 ** 16, size=(L, H, D), dtype=np.uint16)
    val = rng.integers(0, 2 ** 16, size=(L, H, D), dtype=np.uint16)
    nk, nv = oracle.kv_cache_append(kc, vc, key, val, slots, bs)
    assert np.array_equal(oracle.gather_sequence(nk, table, L), key)
    assert np.array_equal(oracle.gather_sequence(nv, table, L), val)
    # rows outside the written slots keep their old bytes
    mask = np.ones((NB, bs), dtype=bool)
    for sl in slots:
        mask[sl // bs, sl % bs] = False
    assert np.array_equal(nk[mask], kc[mask]) and np.array_equal(nv[mask], vc[mask])


def test_append_negative_slot_writes_nothing():
    kc = np.arange(2 * 2 * 1 * 3, dtype=np.float32).reshape(2, 2, 1, 3)
    nk, nv = oracle.kv_cache_append(kc, kc, -np.ones((2, 1, 3), np.float32),
                                    -np.ones((2, 1, 3), np.float32), [-1, -7], 2)
    assert np.array_equal(nk, kc) and np.array_equal(nv, kc)


def test_gather_planted_index_mistake_is_caught():
    # a gather that swaps block index and offset disagrees with the fixture
    fx = _load("kv_append_worked.json")
    nk = np.array(fx["expected_k_cache"], dtype=np.float32)
    g = fx["gather"]
    bad = np.stack([nk[t % 2, int(g["block_table"][t // 2]) % 2] for t in range(g["context_len"])])
    assert not np.array_equal(bad, np.array(g["expected_k"], dtype=np.float32))


# ------------------------------------------------------------------ block manager
def _run_op(bm, op):
    kind = op["op"]
    if kind == "allocate":
        return {"blocks": bm.allocate(op["seq"], op["n"])}
    if kind == "extend":
        slots, cows = bm.extend(op["seq"], op["n"])
        return {"slots": slots, "cow": [list(c) for c in cows]}
    if kind == "fork":
        bm.fork(op["parent"], op["child"])
        return {}
    if kind == "free":
        bm.free(op["seq"])
        return {}
    raise ValueError(kind)


def test_block_manager_matches_hand_worked_history():
    fx = _load("block_manager_worked.json")
    bm = BlockManager(fx["num_blocks"], fx["block_size"], fx["free_order"])
    for i, op in enumerate(fx["ops"], start=1):
        if "error" in op["expect"]:
            before = (list(bm.free_blocks), list(bm.ref_count),
                      {k: list(v) for k, v in bm.block_tables.items()}, dict(bm.num_tokens))
            with pytest.raises(OutOfBlocks):
                _run_op(bm, op)
            after = (list(bm.free_blocks), list(bm.ref_count),
                     {k: list(v) for k, v in bm.block_tables.items()}, dict(bm.num_tokens))
            assert before == after, f"op {i} changed state while failing"
        else:
            assert _run_op(bm, op) == op["expect"], f"op {i}"
        assert bm.free_blocks == op["free_after"], f"free list after op {i}"
        key = f"after_op_{i}"
        if key in fx["tables_after"]:
            assert {str(k): v for k, v in bm.block_tables.items()} == fx["tables_after"][key]
            assert bm.ref_count == fx["ref_counts_after"][key]
    assert {str(k): v for k, v in bm.block_tables.items()} == fx["tables_after"]["final"]
    assert bm.ref_count == fx["ref_counts_after"]["final"]
    assert {str(k): v for k, v in bm.num_tokens.items()} == fx["context_lens_final"]


def test_allocate_takes_ceil_div_blocks_from_the_end():
    bm = BlockManager(10, 16, list(range(10)))
    assert bm.allocate(0, 0) == []
    assert bm.allocate(1, 16) == [9]
    assert bm.allocate(2, 17) == [8, 7]
    assert bm.allocate(3, 33) == [6, 5, 4]
    assert bm.num_free() == 4
    with pytest.raises(OutOfBlocks):
        bm.allocate(4, 16 * 5)
    assert bm.num_free() == 4 and 4 not in bm.block_tables


def _check_invariants(bm: BlockManager):
    NB = bm.num_blocks
    counts = [0] * NB
    for t in bm.block_tables.values():
        for b in t:
            counts[b] += 1
    # ref count == number of tables holding the block; free exactly when unreferenced
    assert counts == bm.ref_count
    free = set(bm.free_blocks)
    assert len(free) == len(bm.free_blocks)
    assert free == {b for b in range(NB) if counts[b] == 0}
    # table length matches the token count
    for s, t in bm.block_tables.items():
        assert len(t) == -(-bm.num_tokens[s] // bm.block_size)


_ops = st.lists(st.tuples(st.sampled_from(["allocate", "extend", "fork", "free"]),
                          st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)),
                max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops=_ops, nb=st.integers(1, 24), bs=st.sampled_from([1, 2, 4, 16]),
       seed=st.integers(0, 1000))
def test_block_manager_invariants_random_histories(ops, nb, bs, seed):
    order = list(np.random.default_rng(seed).permutation(nb))
    bm = BlockManager(nb, bs, order)
    written = {}  # slot -> seq that last wrote it; a slot is never live in two sequences
    for kind, a, b, n in ops:
        snapshot = (list(bm.free_blocks), list(bm.ref_count),
                    {k: list(v) for k, v in bm.block_tables.items()}, dict(bm.num_tokens))
        try:
            if kind == "allocate":
                bm.allocate(a, n)
            elif kind == "extend":
                slots, cows = bm.extend(a, n)
                table = bm.block_tables[a]
                L = bm.num_tokens[a]
                # the new tokens sit where the table says tokens L-n .. L-1 live
                for i, slot in enumerate(slots):
                    t = L - n + i
                    assert slot == table[t // bs] * bs + t % bs
                    assert bm.ref_count[table[t // bs]] == 1  # never write a shared block
                for src, dst in cows:
                    assert bm.ref_count[dst] == 1
            elif kind == "fork":
                bm.fork(a, b)
            else:
                bm.free(a)
        except (KeyError, OutOfBlocks):
            after = (list(bm.free_blocks), list(bm.ref_count),
                     {k: list(v) for k, v in bm.block_tables.items()}, dict(bm.num_tokens))
            assert after == snapshot  # failures are all-or-nothing
        _check_invariants(bm)
