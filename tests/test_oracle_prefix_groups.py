"""CPU pins of the oracle's prefix grouping (``BlockManager.prefix_groups``): the hand-worked
fixture, a token-by-token brute force written from the definition (prefix sharing by
reference to the same physical blocks -- the yunthe.com page, section
"PagedAttention分页注意力机制原理"; the 111cn.net page §3.2), invariants of every group, and
planted mistakes that each of them must catch."""

import json
import os

import numpy as np
import pytest

from oracle.block_manager import BlockManager

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle(bm, seqs, min_prefix=0):
    return bm.prefix_groups(seqs, min_prefix)


# ------------------------------------------------------------------ references
def groups_brute(bm, seqs, min_prefix=0):
    """Token by token: an entry joins the bucket of the block holding its token 0 when that
    block is full; a bucket of two or more shares every leading token t that lies in a full
    block of every member and in the same block id for every member; the shared count is cut
    down to a multiple of 16 and must reach max(16, min_prefix)."""
    bs = bm.block_size
    tab = [bm.block_table(s) for s in seqs]
    lens = [bm.context_len(s) for s in seqs]

    def full_at(i, t):
        return (t // bs + 1) * bs <= lens[i]

    buckets = {}
    for i in range(len(seqs)):
        if full_at(i, 0):
            buckets.setdefault(tab[i][0], []).append(i)
    sp, groups = [0] * len(seqs), []
    for mem in buckets.values():
        if len(mem) < 2:
            continue
        t = 0
        while all(full_at(i, t) and tab[i][t // bs] == tab[mem[0]][t // bs] for i in mem):
            t += 1
        P = t // 16 * 16
        if P < max(16, min_prefix):
            continue
        for i in mem:
            sp[i] = P
        groups.append(mem)
    return sp, groups


def _random_history(seed, bs):
    """Forked families (some with a partly filled shared last block, some extended), lone
    sequences, and families whose root is released; the batch in a shuffled order with some
    members left out."""
    rng = np.random.default_rng(seed)
    bm = BlockManager(600, bs, rng.permutation(600).tolist())
    sid, batch = 0, []
    for fam in range(int(rng.integers(1, 6))):
        root = 10_000 + fam
        bm.allocate(root, int(rng.integers(0, 100)))
        for _ in range(int(rng.integers(1, 5))):
            bm.fork(root, sid)
            if rng.random() < 0.7:
                bm.extend(sid, int(rng.integers(0, 50)))
            batch.append(sid)
            sid += 1
        if rng.random() < 0.5:
            bm.free(root)
        else:
            batch.append(root)
    for _ in range(int(rng.integers(0, 4))):
        bm.allocate(sid, int(rng.integers(0, 60)))
        batch.append(sid)
        sid += 1
    order = rng.permutation(len(batch)).tolist()
    keep = [batch[i] for i in order if rng.random() < 0.9]
    return bm, keep


# ------------------------------------------------------------------ pins
def pin_fixture(impl):
    with open(os.path.join(GOLDEN, "prefix_groups_worked.json"), encoding="utf-8") as f:
        fx = json.load(f)
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
    sp, groups = impl(bm, fx["batch"])
    assert sp == fx["expected_seq_prefix"] and groups == fx["expected_groups"]
    alt = fx["with_min_prefix_tokens_48"]
    sp, groups = impl(bm, fx["batch"], 48)
    assert sp == alt["expected_seq_prefix"] and groups == alt["expected_groups"]


def pin_brute_force(impl, seeds=range(40)):
    for seed in seeds:
        for bs in (8, 16, 32):
            bm, batch = _random_history(seed, bs)
            for min_prefix in (0, 32, 48):
                assert impl(bm, batch, min_prefix) == groups_brute(bm, batch, min_prefix), (seed, bs, min_prefix)


def pin_invariants(impl, seeds=range(40, 70)):
    for seed in seeds:
        for bs in (8, 16, 32):
            bm, batch = _random_history(seed, bs)
            sp, groups = impl(bm, batch)
            grouped = [i for g in groups for i in g]
            assert len(grouped) == len(set(grouped))                 # one group per entry
            assert [g[0] for g in groups] == sorted(g[0] for g in groups)  # ordered by first member
            for i in range(len(batch)):
                if i not in grouped:
                    assert sp[i] == 0
            for g in groups:
                assert len(g) >= 2 and g == sorted(g)
                P = sp[g[0]]
                assert P >= 16 and P % 16 == 0 and all(sp[i] == P for i in g)
                nb = -(-P // bs)
                tabs = [bm.block_table(batch[i]) for i in g]
                assert all(t[:nb] == tabs[0][:nb] for t in tabs)      # the same physical blocks
                assert all(bm.context_len(batch[i]) >= nb * bs for i in g)  # ... each one full


PINS = [pin_fixture, pin_brute_force, pin_invariants]


def test_oracle_passes_every_pin():
    for pin in PINS:
        pin(_oracle)


def test_brute_force_reference_agrees_with_the_fixture():
    pin_fixture(groups_brute)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    def impl(bm, seqs, min_prefix=0):
        bs = bm.block_size
        sp, buckets = [0] * len(seqs), {}
        for i, s in enumerate(seqs):
            tab, n = bm.block_table(s), bm.context_len(s)
            eligible = n >= 1 if kind == "count_partial" else n // bs >= 1
            if eligible and tab:
                buckets.setdefault(tab[-1] if kind == "bucket_by_last" else tab[0], []).append(i)
        groups = []
        for mem in buckets.values():
            if len(mem) < (1 if kind == "singletons" else 2):
                continue
            tabs = [bm.block_table(seqs[i]) for i in mem]
            per = [(-(-bm.context_len(seqs[i]) // bs)) if kind == "count_partial" else bm.context_len(seqs[i]) // bs
                   for i in mem]
            full = min(per)
            k = 0
            while k < full and (kind == "no_compare" or
                                all(k < len(t) and t[k] == tabs[0][k] for t in tabs)):
                k += 1
            tokens = k * bs if kind == "no_round" else k * bs // 16 * 16
            floor = {"no_threshold": 1, "ignore_min_prefix": 16}.get(kind, max(16, min_prefix))
            if tokens < floor:
                continue
            for i in mem:
                sp[i] = tokens
            groups.append(mem)
        return sp, groups

    return impl


# Taking the largest rather than the smallest member's full-block count is no mistake one can
# plant: a block held by several sequences has the same fill for each of them (extend copies a
# shared, partly filled block before writing), so the table comparison stops at the same place.
MUTANTS = ["count_partial", "bucket_by_last", "singletons", "no_compare", "no_round", "no_threshold",
           "ignore_min_prefix"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    impl = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the '{kind}' mistake"


def test_mutant_harness_is_faithful_without_a_mistake():
    for pin in PINS:
        pin(_mutant("none"))
