"""CPU pins of the oracle's whole-block copies (copy-on-write inside a pool, swap between
pools): a hand-worked fixture, the copy-on-write story of a forked sequence told through the
block manager and the append/gather oracle, and properties on random pools."""

import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle.block_manager import BlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    with open(os.path.join(GOLDEN, "block_copy_worked.json"), encoding="utf-8") as f:
        return json.load(f)


def test_copy_matches_hand_worked_fixture():
    fx = _fixture()
    k = np.array(fx["k_pool"], dtype=np.float32)
    v = np.array(fx["v_pool"], dtype=np.float32)
    nk, nv = oracle.copy_blocks(k, v, fx["copy"]["pairs"])
    assert np.array_equal(nk, np.array(fx["copy"]["expected_k"], dtype=np.float32))
    assert np.array_equal(nv, np.array(fx["copy"]["expected_v"], dtype=np.float32))
    assert np.array_equal(k, np.array(fx["k_pool"], dtype=np.float32))  # input untouched
    sk, sv = oracle.copy_blocks(k, v, fx["copy_onto_itself"]["pairs"])
    assert np.array_equal(sk, k) and np.array_equal(sv, v)


def test_swap_matches_hand_worked_fixture():
    fx = _fixture()
    k = np.array(fx["k_pool"], dtype=np.float32)
    v = np.array(fx["v_pool"], dtype=np.float32)
    sw = fx["swap"]
    dk = np.full((sw["dst_blocks"],) + k.shape[1:], sw["fill"], dtype=np.float32)
    dv = dk.copy()
    nk, nv = oracle.swap_blocks(dk, dv, k, v, sw["pairs"])
    assert np.array_equal(nk, np.array(sw["expected_k"], dtype=np.float32))
    assert np.array_equal(nv, np.array(sw["expected_v"], dtype=np.float32))


def test_copy_on_write_keeps_parent_and_extends_child():
    """A parent with a partly filled last block is forked; the child appends one token.  The
    block manager reports one (shared, fresh) pair; after the copy and the child's append the
    parent reads back its own tokens and the child reads the parent's tokens plus its new one.
    A missing copy, a reversed copy or a partial copy each break one of these reads."""
    rng = np.random.default_rng(3)
    bs, hkv, d = 16, 2, 4
    bm = BlockManager(8, bs, free_order=rng.permutation(8).tolist())
    k = np.full((8, bs, hkv, d), np.nan, dtype=np.float32)
    v = k.copy()
    parent_k = rng.standard_normal((20, hkv, d)).astype(np.float32)
    parent_v = rng.standard_normal((20, hkv, d)).astype(np.float32)
    bm.allocate(0, 0)
    slots, cows = bm.extend(0, 20)
    assert cows == []
    k, v = oracle.kv_cache_append(k, v, parent_k, parent_v, slots, bs)
    bm.fork(0, 1)
    new_k = rng.standard_normal((1, hkv, d)).astype(np.float32)
    new_v = rng.standard_normal((1, hkv, d)).astype(np.float32)
    slots, cows = bm.extend(1, 1)
    assert len(cows) == 1
    src, dst = cows[0]
    assert bm.block_table(0)[-1] == src and bm.block_table(1)[-1] == dst and src != dst
    k, v = oracle.copy_blocks(k, v, cows)
    k, v = oracle.kv_cache_append(k, v, new_k, new_v, slots, bs)
    got_pk = oracle.gather_sequence(k, bm.block_table(0), bm.context_len(0))
    got_pv = oracle.gather_sequence(v, bm.block_table(0), bm.context_len(0))
    assert np.array_equal(got_pk, parent_k) and np.array_equal(got_pv, parent_v)
    got_ck = oracle.gather_sequence(k, bm.block_table(1), bm.context_len(1))
    got_cv = oracle.gather_sequence(v, bm.block_table(1), bm.context_len(1))
    assert np.array_equal(got_ck, np.concatenate([parent_k, new_k]))
    assert np.array_equal(got_cv, np.concatenate([parent_v, new_v]))


@settings(max_examples=60, deadline=None)
@given(st.integers(min_value=2, max_value=12), st.integers(min_value=0, max_value=2**31 - 1),
       st.integers(min_value=0, max_value=6))
def test_copy_properties(nb, seed, n_pairs):
    """Destinations hold their source's old data; every other block is untouched."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((nb, 3, 2, 2)).astype(np.float32)
    v = rng.standard_normal((nb, 3, 2, 2)).astype(np.float32)
    perm = rng.permutation(nb).tolist()
    n = min(n_pairs, nb // 2)
    srcs, dsts = perm[:n], perm[n:2 * n]  # disjoint: no destination is also a source
    pairs = list(zip(srcs, dsts))
    nk, nv = oracle.copy_blocks(k, v, pairs)
    for b in range(nb):
        if b in dsts:
            s = srcs[dsts.index(b)]
            assert np.array_equal(nk[b], k[s]) and np.array_equal(nv[b], v[s])
        else:
            assert np.array_equal(nk[b], k[b]) and np.array_equal(nv[b], v[b])


@settings(max_examples=40, deadline=None)
@given(st.integers(min_value=1, max_value=10), st.integers(min_value=0, max_value=2**31 - 1))
def test_swap_out_and_back_restores_blocks(nb, seed):
    """Blocks swapped out to a host pool at fresh ids and back in at other ids read back equal."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((nb, 2, 1, 3)).astype(np.float32)
    v = rng.standard_normal((nb, 2, 1, 3)).astype(np.float32)
    chosen = rng.permutation(nb)[: rng.integers(1, nb + 1)].tolist()
    host_ids = rng.permutation(len(chosen) + 3)[: len(chosen)].tolist()
    k0 = k.copy()
    hk = np.zeros((len(chosen) + 3,) + k.shape[1:], dtype=np.float32)
    hv = hk.copy()
    hk, hv = oracle.swap_blocks(hk, hv, k, v, list(zip(chosen, host_ids)))
    back_ids = rng.permutation(nb)[: len(chosen)].tolist()
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dk, dv = oracle.swap_blocks(dk, dv, hk, hv, list(zip(host_ids, back_ids)))
    for c, b in zip(chosen, back_ids):
        assert np.array_equal(dk[b], k[c]) and np.array_equal(dv[b], v[c])
    assert np.array_equal(k, k0)  # the source pool is only read


# ------------------------------------------------------------------ swap of whole sequences
def _swap_fixture():
    with open(os.path.join(GOLDEN, "block_swap_worked.json"), encoding="utf-8") as f:
        return json.load(f)


def _setup_pools(fx):
    d = BlockManager(fx["device_pool"]["num_blocks"], fx["device_pool"]["block_size"], fx["device_pool"]["free_order"])
    h = BlockManager(fx["host_pool"]["num_blocks"], fx["host_pool"]["block_size"], fx["host_pool"]["free_order"])
    for op in fx["setup"]:
        if op["op"] == "allocate":
            d.allocate(op["seq"], op["tokens"])
        elif op["op"] == "fork":
            d.fork(op["parent"], op["child"])
        else:
            d.extend(op["seq"], op["n"])
    return d, h


def test_move_seqs_matches_hand_worked_fixture():
    import pytest
    from oracle.block_manager import SharedWithStayingSequence

    fx = _swap_fixture()
    d, h = _setup_pools(fx)
    with pytest.raises(SharedWithStayingSequence):
        d.move_seqs(h, fx["refused"]["seqs"])
    assert d.free_blocks == [0, 1] and h.free_blocks == [0, 1, 2, 3]  # nothing changed
    out = fx["out"]
    assert [list(p) for p in d.move_seqs(h, out["seqs"])] == out["expected_pairs"]
    assert {str(k): v for k, v in h.block_tables.items()} == out["expected_host_tables"]
    assert {str(b): h.ref_count[b] for b in range(4) if h.ref_count[b]} == out["expected_host_refs"]
    assert h.free_blocks == out["expected_host_free"] and d.free_blocks == out["expected_device_free"]
    assert {str(k): v for k, v in d.block_tables.items()} == out["expected_device_tables"]
    back = fx["back"]
    assert [list(p) for p in h.move_seqs(d, back["seqs"])] == back["expected_pairs"]
    assert {str(k): v for k, v in d.block_tables.items()} == back["expected_device_tables"]
    assert d.free_blocks == back["expected_device_free"] and h.free_blocks == back["expected_host_free"]


@settings(max_examples=40, deadline=None)
@given(st.integers(min_value=0, max_value=2**31 - 1))
def test_swap_out_and_in_keeps_every_sequence_readable(seed):
    """Random sequences (some forked, some extended with copy-on-write) swap out to a host pool
    and back with the block copies of ``swap_blocks``: every sequence gathers the same rows as
    before, and reference counts match the tables."""
    rng = np.random.default_rng(seed)
    bs, hkv, d = 4, 1, 2
    dev = BlockManager(24, bs, rng.permutation(24).tolist())
    host = BlockManager(20, bs, rng.permutation(20).tolist())
    dk = rng.standard_normal((24, bs, hkv, d)).astype(np.float32)
    dv = rng.standard_normal((24, bs, hkv, d)).astype(np.float32)
    hk = np.full((20, bs, hkv, d), np.nan, dtype=np.float32)
    hv = hk.copy()
    dev.allocate(0, int(rng.integers(1, 9)))
    dev.fork(0, 1)
    slots, cows = dev.extend(1, int(rng.integers(0, 3)))
    dk, dv = oracle.copy_blocks(dk, dv, cows)
    dev.allocate(2, int(rng.integers(0, 7)))
    before = {s: (oracle.gather_sequence(dk, dev.block_table(s), dev.context_len(s)),
                  oracle.gather_sequence(dv, dev.block_table(s), dev.context_len(s))) for s in (0, 1, 2)}
    moving = [[0, 1], [2], [1, 0, 2]][int(rng.integers(0, 3))]
    pairs = dev.move_seqs(host, moving)
    hk, hv = oracle.swap_blocks(hk, hv, dk, dv, pairs)
    dk = np.where(np.isnan(dk), dk, dk + 1000)  # the device pool's old data is dead once moved
    dv = np.where(np.isnan(dv), dv, dv + 1000)
    for s in (0, 1, 2):
        if s in moving:
            assert oracle.gather_sequence(hk, host.block_table(s), host.context_len(s)).tolist() == before[s][0].tolist()
    back = host.move_seqs(dev, moving)
    dk, dv = oracle.swap_blocks(dk, dv, hk, hv, back)
    for s in moving:
        assert np.array_equal(oracle.gather_sequence(dk, dev.block_table(s), dev.context_len(s)), before[s][0])
        assert np.array_equal(oracle.gather_sequence(dv, dev.block_table(s), dev.context_len(s)), before[s][1])
    for pool in (dev, host):
        refs = [0] * pool.num_blocks
        for t in pool.block_tables.values():
            for b in t:
                refs[b] += 1
        assert refs == pool.ref_count
        assert sorted(pool.free_blocks + [b for b in range(pool.num_blocks) if refs[b]]) == list(range(pool.num_blocks))


# ------------------------------------------------------------------ prefix groups
def _replay(fx):
    bm = BlockManager(fx["num_blocks"], fx["block_size"])
    for op in fx["ops"]:
        if op["op"] == "allocate":
            bm.allocate(op["seq"], op["tokens"])
        elif op["op"] == "fork":
            bm.fork(op["parent"], op["child"])
        elif op["op"] == "free":
            bm.free(op["seq"])
        else:
            bm.extend(op["seq"], op["n"])
    return bm


def test_prefix_groups_match_hand_worked_fixture():
    with open(os.path.join(GOLDEN, "prefix_groups_worked.json"), encoding="utf-8") as f:
        fx = json.load(f)
    bm = _replay(fx)
    sp, groups = bm.prefix_groups(fx["batch"])
    assert sp == fx["expected_seq_prefix"] and groups == fx["expected_groups"]
    alt = fx["with_min_prefix_tokens_48"]
    sp, groups = bm.prefix_groups(fx["batch"], 48)
    assert sp == alt["expected_seq_prefix"] and groups == alt["expected_groups"]


@settings(max_examples=80, deadline=None)
@given(st.integers(min_value=0, max_value=2**31 - 1), st.sampled_from([8, 16, 32]))
def test_prefix_groups_are_shared_and_maximal(seed, bs):
    """Forked families with random suffixes: every group's members name the same blocks for the
    first P tokens, P is a multiple of 16 covered by full blocks of every member, and a group's
    common run of full shared blocks is not longer than P rounds down from."""
    rng = np.random.default_rng(seed)
    bm = BlockManager(400, bs, rng.permutation(400).tolist())
    batch, sid = [], 0
    for fam in range(int(rng.integers(1, 5))):
        root = 10_000 + fam
        bm.allocate(root, int(rng.integers(0, 120)))
        for _ in range(int(rng.integers(1, 5))):
            bm.fork(root, sid)
            bm.extend(sid, int(rng.integers(0, 40)))
            batch.append(sid)
            sid += 1
        bm.free(root)
    order = rng.permutation(len(batch)).tolist()
    batch = [batch[i] for i in order]
    sp, groups = bm.prefix_groups(batch)
    grouped = {i for g in groups for i in g}
    for i in range(len(batch)):
        if i not in grouped:
            assert sp[i] == 0
    for g in groups:
        P = sp[g[0]]
        assert P % 16 == 0 and P >= 16 and all(sp[i] == P for i in g) and g == sorted(g)
        nb = P // bs if P % bs == 0 else P // bs + 1
        tabs = [bm.block_table(batch[i]) for i in g]
        assert all(t[:nb] == tabs[0][:nb] for t in tabs)
        assert all(bm.context_len(batch[i]) >= P for i in g)
        full = min(bm.context_len(batch[i]) // bs for i in g)
        k = 0
        while k < full and all(t[k] == tabs[0][k] for t in tabs):
            k += 1
        assert P == k * bs // 16 * 16
