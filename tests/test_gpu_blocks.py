"""GPU tests of the whole-block copies through the C ABI (pkv_copy_blocks, pkv_swap_blocks):
bit-exact against the oracle's copies on pools with NaN canaries, the copy-on-write path of a
forked sequence end to end (decode of parent and child against the attention oracle), and
swap through pinned host memory."""

import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import BlockManager
from paged_kv_cache_376_amd import binding
from paged_kv_cache_376_amd.cache import PagedKVCache
from tests.gpu_common import DEVICE, TOL, decode, max_err, say

pytestmark = pytest.mark.gpu

SHAPES = [("bfloat16", 16, 8, 128), ("float16", 16, 2, 64), ("float32", 16, 4, 64), ("bfloat16", 16, 1, 128)]


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view({4: torch.int32, 2: torch.int16}[t.element_size()]).numpy()


def _random_pool(rng, nb, bs, hkv, d, dtype):
    x = torch.from_numpy(rng.standard_normal((nb, bs, hkv, d), dtype=np.float32)).to(getattr(torch, dtype))
    x[rng.integers(0, nb, size=max(1, nb // 8))] = float("nan")  # some blocks hold NaN canaries
    return x


def _pairs(rng, nb, n):
    perm = rng.permutation(nb).tolist()
    srcs, dsts = perm[:n], perm[n:2 * n]  # no destination is also a source
    untouched = perm[2 * n]
    # plus pairs the call must skip: ids outside the pool and a block onto itself
    return list(zip(srcs, dsts)) + [(nb, dsts[0]), (-1, dsts[0]), (srcs[0], nb + 7), (untouched, untouched)]


@pytest.mark.parametrize("shape", SHAPES)
def test_copy_blocks_matches_oracle(shape):
    dtype, bs, hkv, d = shape
    say(f"[copy_blocks] {shape}")
    rng = np.random.default_rng(21)
    nb = 64
    k = _random_pool(rng, nb, bs, hkv, d, dtype)
    v = _random_pool(rng, nb, bs, hkv, d, dtype)
    pairs = _pairs(rng, nb, 20)
    ek, ev = oracle.copy_blocks(_bits(k), _bits(v), pairs)
    kd, vd = k.to(DEVICE), v.to(DEVICE)
    binding.copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device=DEVICE))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kd), ek) and np.array_equal(_bits(vd), ev)


def test_copy_blocks_more_pairs_than_one_grid_column():
    """More pairs than the launch's pair groups (65535): work-groups stride over pairs."""
    say("[copy_blocks] 70000 pairs")
    rng = np.random.default_rng(22)
    nb, n = 140_100, 70_000
    k = torch.from_numpy(rng.integers(-30000, 30000, size=(nb, 16, 1, 64), dtype=np.int16))
    v = torch.from_numpy(rng.integers(-30000, 30000, size=(nb, 16, 1, 64), dtype=np.int16))
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32)
    ek, ev = k.numpy().copy(), v.numpy().copy()
    ek[pairs[:, 1]] = k.numpy()[pairs[:, 0]]
    ev[pairs[:, 1]] = v.numpy()[pairs[:, 0]]
    kd, vd = k.view(torch.float16).to(DEVICE), v.view(torch.float16).to(DEVICE)
    binding.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEVICE))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kd), ek) and np.array_equal(_bits(vd), ev)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bfloat16", 16, 2, 128), ("float16", 8, 8, 64), ("float32", 4, 4, 64)])
def test_copy_on_write_fork_then_decode(dtype, hq, hkv, d):
    """Parent with a partly filled last block, forked; the child appends one token (its shared
    last block is copied by pkv_copy_blocks first).  Both decode to the oracle, the parent's
    blocks are bit-for-bit unchanged, and the host pool agrees with the oracle's manager."""
    say(f"[cow decode] {dtype} Hq={hq} Hkv={hkv} D={d}")
    tdt = getattr(torch, dtype)
    rng = np.random.default_rng(23)
    order = rng.permutation(16).astype(np.int32)
    cache = PagedKVCache(16, hkv, d, tdt, DEVICE, free_order=order, fill=float("nan"))
    bm = BlockManager(16, 16, free_order=order.tolist())
    kp = torch.from_numpy(rng.standard_normal((37, hkv, d), dtype=np.float32)).to(tdt)
    vp = torch.from_numpy(rng.standard_normal((37, hkv, d), dtype=np.float32)).to(tdt)
    cache.add_sequence(0, kp, vp)
    bm.allocate(0, 0)
    bm.extend(0, 37)
    parent_blocks = bm.block_table(0)
    before_k = _bits(cache.k_cache[parent_blocks])
    cache.fork(0, 1)
    bm.fork(0, 1)
    kn = torch.from_numpy(rng.standard_normal((1, hkv, d), dtype=np.float32)).to(tdt)
    vn = torch.from_numpy(rng.standard_normal((1, hkv, d), dtype=np.float32)).to(tdt)
    slots = cache.extend(1, kn, vn)
    oslots, cows = bm.extend(1, 1)
    assert slots.tolist() == oslots and len(cows) == 1
    assert np.array_equal(_bits(cache.k_cache[parent_blocks]), before_k)
    q = torch.from_numpy(rng.standard_normal((2, hq, d), dtype=np.float32)).to(tdt)
    bt, ctx, maxc = cache.tables([0, 1])
    out = decode(cache, q, bt, ctx, maxc, 1.0 / np.sqrt(d), 0)
    ref = oracle.decode_attention(q, [kp, torch.cat([kp, kn])], [vp, torch.cat([vp, vn])], 1.0 / np.sqrt(d))
    err = max_err(out, ref)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("pairs_on_host", [False, True])
def test_swap_round_trip_through_pinned_host(pairs_on_host):
    """Blocks go out to pinned host pools at fresh ids and come back to other device ids;
    every destination matches the oracle's swap bit for bit and nothing else is written."""
    say(f"[swap] pairs on host {pairs_on_host}")
    rng = np.random.default_rng(24)
    nb, nh = 48, 40
    shape = (16, 8, 128)
    k = _random_pool(rng, nb, *shape, "bfloat16")
    v = _random_pool(rng, nb, *shape, "bfloat16")
    kd, vd = k.to(DEVICE), v.to(DEVICE)
    hk = torch.full((nh,) + shape, float("nan"), dtype=torch.bfloat16).pin_memory()
    hv = torch.full((nh,) + shape, float("nan"), dtype=torch.bfloat16).pin_memory()
    chosen = rng.permutation(nb)[:30].tolist()
    host_ids = rng.permutation(nh)[:30].tolist()
    out_pairs = list(zip(chosen, host_ids)) + [(nb, 0), (0, nh)]

    def pairs_tensor(p):
        t = torch.tensor(p, dtype=torch.int32)
        return t.pin_memory() if pairs_on_host else t.to(DEVICE)

    ehk, ehv = oracle.swap_blocks(_bits(hk), _bits(hv), _bits(k), _bits(v), out_pairs)
    binding.swap_blocks(hk, hv, kd, vd, pairs_tensor(out_pairs))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(hk), ehk) and np.array_equal(_bits(hv), ehv)
    assert np.array_equal(_bits(kd), _bits(k))  # the source is only read
    back = torch.full((nb,) + shape, float("nan"), dtype=torch.bfloat16, device=DEVICE)
    back_v = back.clone()
    back_ids = rng.permutation(nb)[:30].tolist()
    in_pairs = list(zip(host_ids, back_ids))
    ebk, ebv = oracle.swap_blocks(_bits(back), _bits(back_v), ehk, ehv, in_pairs)
    binding.swap_blocks(back, back_v, hk, hv, pairs_tensor(in_pairs))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), ebk) and np.array_equal(_bits(back_v), ebv)
    for c, b in zip(chosen, back_ids):
        assert np.array_equal(_bits(back[b]), _bits(k[c]))


def test_swap_refuses_pageable_host_memory():
    """A host pool that is not pinned is refused before any launch; nothing is written."""
    say("[swap] pageable host memory refused")
    shape = (4, 16, 2, 64)
    kd = torch.zeros(shape, dtype=torch.float16, device=DEVICE)
    vd = torch.zeros(shape, dtype=torch.float16, device=DEVICE)
    hk = torch.ones(shape, dtype=torch.float16)
    hv = torch.ones(shape, dtype=torch.float16)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device=DEVICE)
    with pytest.raises(binding.PkvError) as ei:
        binding.swap_blocks(kd, vd, hk, hv, pairs)
    assert ei.value.status == 1
    torch.cuda.synchronize()
    assert torch.count_nonzero(kd).item() == 0 and torch.count_nonzero(vd).item() == 0


def test_sequences_swap_out_and_back_decode_bitwise_equal():
    """Sequences (two of them sharing a forked prefix) move to a pinned host cache, their device
    blocks are reused and overwritten by another sequence, and they move back to other block
    ids: decode gives bit-for-bit the output from before (the block-relabel invariance), which
    also matches the attention oracle."""
    say("[swap seqs] out, overwrite, back, decode")
    rng = np.random.default_rng(25)
    tdt, hq, hkv, d = torch.bfloat16, 16, 2, 128
    dev = PagedKVCache(64, hkv, d, tdt, DEVICE, free_order=rng.permutation(64).astype(np.int32), fill=float("nan"))
    host = PagedKVCache(48, hkv, d, tdt, "cpu", free_order=rng.permutation(48).astype(np.int32), fill=float("nan"),
                        pinned=True)
    kv = {}
    for s, L in ((0, 50), (1, 200), (2, 17)):
        k = torch.from_numpy(rng.standard_normal((L, hkv, d), dtype=np.float32)).to(tdt)
        v = torch.from_numpy(rng.standard_normal((L, hkv, d), dtype=np.float32)).to(tdt)
        dev.add_sequence(s, k, v)
        kv[s] = (k, v)
    dev.fork(1, 3)  # 3 shares 1's 13 blocks; its own token goes through copy-on-write
    kn = torch.from_numpy(rng.standard_normal((5, hkv, d), dtype=np.float32)).to(tdt)
    vn = torch.from_numpy(rng.standard_normal((5, hkv, d), dtype=np.float32)).to(tdt)
    dev.extend(3, kn, vn)
    kv[3] = (torch.cat([kv[1][0], kn]), torch.cat([kv[1][1], vn]))
    seqs = [0, 1, 2, 3]
    q = torch.from_numpy(rng.standard_normal((4, hq, d), dtype=np.float32)).to(tdt)
    bt, ctx, maxc = dev.tables(seqs)
    first = decode(dev, q, bt, ctx, maxc, 0.088, 0)
    pairs = dev.move_to(host, [1, 3, 2])
    assert len(pairs) == 13 + 1 + 2 and dev.pool.num_seqs() == 1
    junk = torch.full((600, hkv, d), 3.0, dtype=tdt)  # takes (and overwrites) the freed blocks
    dev.add_sequence(9, junk, junk)
    dev.pool.seq_free(9)
    back = host.move_to(dev, [3, 1, 2])
    assert len(back) == len(pairs) and host.pool.num_seqs() == 0
    bt2, ctx2, maxc2 = dev.tables(seqs)
    assert not torch.equal(bt2.cpu(), bt.cpu())  # other physical blocks
    second = decode(dev, q, bt2, ctx2, maxc2, 0.088, 0)
    assert torch.equal(first.view(torch.int16), second.view(torch.int16))
    ref = oracle.decode_attention(q, [kv[s][0] for s in seqs], [kv[s][1] for s in seqs], 0.088)
    err = max_err(second, ref)
    say(f"    max abs err {err:.3e}")
    assert err <= TOL["bfloat16"]


def _int_pool(rng, nb, shape):
    return torch.from_numpy(rng.integers(-32768, 32767, size=(nb,) + shape, dtype=np.int16, endpoint=True))


def test_copy_blocks_bench_size():
    """The benchmark's copy (bench.py --op copy_blocks): 4096 pairs of 16 x 8 x 128 bf16 blocks
    in a 16384-block pool, bit for bit against the oracle's copy over the whole pool."""
    say("[copy_blocks] bench size: 4096 pairs, 16384 blocks of 32 KiB")
    rng = np.random.default_rng(0)
    nb, n, shape = 16384, 4096, (16, 8, 128)
    k, v = _int_pool(rng, nb, shape), _int_pool(rng, nb, shape)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32)
    ek, ev = oracle.copy_blocks(k.numpy(), v.numpy(), pairs.tolist())
    kd, vd = k.view(torch.bfloat16).to(DEVICE), v.view(torch.bfloat16).to(DEVICE)
    binding.copy_blocks(kd, vd, torch.from_numpy(pairs).to(DEVICE))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kd), ek) and np.array_equal(_bits(vd), ev)


def test_swap_bench_size():
    """The benchmark's swap (bench.py --op swap): 2048 blocks of 32 KiB from an 8192-block
    device pool out to a 4096-block pinned host pool and back to other device ids, bit for bit
    against the oracle's swaps."""
    say("[swap] bench size: 2048 blocks out and back")
    rng = np.random.default_rng(1)
    nb, nh, n, shape = 8192, 4096, 2048, (16, 8, 128)
    k, v = _int_pool(rng, nb, shape), _int_pool(rng, nb, shape)
    kd, vd = k.view(torch.bfloat16).to(DEVICE), v.view(torch.bfloat16).to(DEVICE)
    hk0, hv0 = _int_pool(rng, nh, shape), _int_pool(rng, nh, shape)
    hk, hv = hk0.view(torch.bfloat16).pin_memory(), hv0.view(torch.bfloat16).pin_memory()
    dev_ids = rng.permutation(nb)[:n]
    host_ids = rng.permutation(nh)[:n]
    out_pairs = np.stack([dev_ids, host_ids], axis=1).astype(np.int32)
    ehk, ehv = oracle.swap_blocks(hk0.numpy(), hv0.numpy(), k.numpy(), v.numpy(), out_pairs.tolist())
    binding.swap_blocks(hk, hv, kd, vd, torch.from_numpy(out_pairs).to(DEVICE))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(hk), ehk) and np.array_equal(_bits(hv), ehv)
    back_ids = rng.permutation(nb)[:n]
    in_pairs = np.stack([host_ids, back_ids], axis=1).astype(np.int32)
    ebk, ebv = oracle.swap_blocks(k.numpy(), v.numpy(), ehk, ehv, in_pairs.tolist())
    binding.swap_blocks(kd, vd, hk, hv, torch.from_numpy(in_pairs).to(DEVICE))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kd), ebk) and np.array_equal(_bits(vd), ebv)
