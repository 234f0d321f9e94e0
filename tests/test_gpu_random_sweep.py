"""GPU parity over seeded random points of the argument space, against the fp64 oracle.

Each case draws (from its own seed) the element type, head dim, KV heads, group size, batch,
length mix (lognormal, uniform, with empty contexts), block size, partition size and whether
the append is fused into the decode, then compares every output of every sequence with the
oracle (and, for the fused call, every appended row bit for bit).  A second set draws
prefix-shared batches (group sizes, prefix lengths that end inside a block, empty suffixes,
ungrouped sequences) for pkv_paged_attn_decode_prefix.  Sizes stay where the oracle takes a
second or two.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_376_amd import binding
from paged_kv_cache_376_amd import workloads as W
from paged_kv_cache_376_amd.cache import build_cache
from tests.gpu_common import DEVICE, TOL, decode_step, decode_step_fused, max_err, oracle_out, say

pytestmark = pytest.mark.gpu


def _draw(seed, hkv_choices=(1, 2, 3, 4, 5, 8)):
    rng = np.random.default_rng(seed)
    dtype = rng.choice(["bfloat16", "float16", "float32"], p=[0.5, 0.35, 0.15])
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice(hkv_choices))
    g = int(rng.choice([1, 2])) if dtype == "float32" else int(rng.choice([1, 1, 2, 3, 4, 5, 7, 8, 8, 9, 12, 16]))
    b = int(rng.choice([1, 2, 3, 5, 7, 8, 9, 17, 40, 130, 300]))
    # about 1.5M (token x KV head) pairs at most, so that the oracle stays fast
    cap = max(16, min(6000, int(1.5e6 / (b * hkv))))
    kind = rng.choice(["lognormal", "uniform", "zeros"])
    if kind == "lognormal":
        lens = np.clip(np.round(cap / 4 * np.exp(rng.standard_normal(b))), 0, cap)
    elif kind == "uniform":
        lens = rng.integers(0, cap + 1, size=b)
    else:
        lens = rng.integers(0, cap + 1, size=b) * (rng.random(b) < 0.6)
    partition = int(rng.choice([0, -1, 16, 48, 256], p=[0.6, 0.1, 0.1, 0.1, 0.1]))
    bs = 16 if (dtype == "float32" or partition != 0) else int(rng.choice([8, 16, 32]))
    fused = bool(rng.random() < 0.5)
    spec = W.Spec(f"rand{seed}", str(dtype), b, g * hkv, hkv, d, "fixed",
                  fixed_lengths=tuple(int(x) for x in lens), block_size=bs)
    return spec, partition, fused


@pytest.mark.parametrize("seed", range(48))
def test_random_decode_matches_oracle(seed):
    _check_decode(seed, *_draw(1000 + seed))


@pytest.mark.parametrize("seed", range(8))
def test_random_decode_many_kv_heads(seed):
    """12 to 32 KV heads: 3 to 8 groups of 4 heads per range (with one query head per KV
    head, the work-groups take two pairs of heads from the two halves of the head range)."""
    _check_decode(200 + seed, *_draw(4000 + seed, hkv_choices=(12, 16, 20, 24, 32)))


def _check_decode(seed, spec, partition, fused):
    say(f"[random] seed {seed}: {spec.dtype} D={spec.head_dim} Hkv={spec.num_kv_heads} "
        f"G={spec.num_q_heads // spec.num_kv_heads} B={spec.num_seqs} bs={spec.block_size} "
        f"partition={partition} fused={fused} max len={max(spec.fixed_lengths)}")
    w = W.Workload(spec, seed=seed)
    if fused:
        out, cache, _, _, _, slots = decode_step_fused(w, partition_size=partition)
    else:
        out, *_ = decode_step(w, partition_size=partition)
    assert torch.isfinite(out.float()).all()
    err = max_err(out, oracle_out(w))
    say(f"    max abs err {err:.3e}")
    assert err <= TOL[spec.dtype], err
    if fused:
        bs = spec.block_size
        sl = torch.from_numpy(slots).to(cache.k_cache.device)
        view = {4: torch.int32, 2: torch.int16}[cache.k_cache.element_size()]
        assert torch.equal(cache.k_cache[sl // bs, sl % bs].cpu().view(view), w.new_k.view(view))
        assert torch.equal(cache.v_cache[sl // bs, sl % bs].cpu().view(view), w.new_v.view(view))


def _draw_prefix(seed, hkv_choices=(1, 2, 4, 8)):
    rng = np.random.default_rng(seed)
    dtype = str(rng.choice(["bfloat16", "float16"]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice(hkv_choices))
    g = int(rng.integers(1, 17))
    gs = int(rng.choice([2, 3, 4, 8]))
    groups = int(rng.integers(1, 9))
    prefix = int(rng.integers(1, 1500))
    suffix_hi = int(rng.choice([0, 20, 300, 900]))
    bs = int(rng.choice([8, 16, 32]))
    spec = W.Spec(f"randp{seed}", dtype, gs * groups, g * hkv, hkv, d, "prefix", prefix_len=prefix,
                  group_size=gs, suffix_lo=0, suffix_hi=suffix_hi, block_size=bs)
    return spec, int(rng.choice([0, 0, 32, 100000]))


@pytest.mark.parametrize("seed", range(16))
def test_random_prefix_decode_matches_oracle(seed):
    _check_prefix(seed, *_draw_prefix(2000 + seed))


@pytest.mark.parametrize("seed", range(8))
def test_random_prefix_decode_partial_head_groups(seed):
    """KV head counts that leave the last group of 4 heads of a work-group partly empty."""
    _check_prefix(100 + seed, *_draw_prefix(3000 + seed, hkv_choices=(3, 5, 6, 7)))


@pytest.mark.parametrize("seed", range(8))
def test_random_prefix_decode_fused_append_matches_oracle(seed):
    """pkv_paged_attn_decode_prefix_append on random shapes: the shuffled batch's sequences
    take their next slots, groups are found on the extended tables, one call appends and
    decodes; every output against the oracle and every new row in its slot bit for bit."""
    _check_prefix(300 + seed, *_draw_prefix(4000 + seed), fused=True)


def _check_prefix(seed, spec, min_prefix, fused=False):
    say(f"[random prefix] seed {seed}: {spec.dtype} D={spec.head_dim} Hkv={spec.num_kv_heads} "
        f"G={spec.num_q_heads // spec.num_kv_heads} groups of {spec.group_size} x {spec.num_seqs // spec.group_size} "
        f"prefix={spec.prefix_len} suffix<= {spec.suffix_hi} bs={spec.block_size} min_prefix={min_prefix}")
    w = W.Workload(spec, seed=seed)
    cache = build_cache(w, DEVICE, fill=float("nan"))
    seqs = list(range(spec.num_seqs))
    # a shuffled batch, with one sequence left out when there are several
    order = list(np.random.default_rng(seed).permutation(spec.num_seqs))
    batch = [int(x) for x in (order[:-1] if len(order) > 2 else order)]
    if fused:  # only the batch's sequences take a slot; the call writes their rows
        slots = []
        for s in batch:
            sl, cow = cache.pool.seq_extend(s, 1)
            cache.copy_blocks(cow)
            slots.append(int(sl[0]))
    else:
        cache.append_tokens(seqs, w.new_k, w.new_v)
    bt, ctx, maxc = cache.tables(batch)
    sp, offs, mem, mx = cache.pool.prefix_groups(batch, min_prefix)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEVICE)
    q = w.q[batch].to(DEVICE).contiguous()
    out = torch.empty_like(q)
    if fused:
        binding.paged_attn_decode_prefix_append(out, q, w.new_k[batch].to(DEVICE).contiguous(),
                                                w.new_v[batch].to(DEVICE).contiguous(), cache.k_cache, cache.v_cache,
                                                bt, ctx, maxc, w.scale, dev(sp), dev(offs), dev(mem), mx)
    else:
        binding.paged_attn_decode_prefix(out, q, cache.k_cache, cache.v_cache, bt, ctx, maxc, w.scale,
                                         dev(sp), dev(offs), dev(mem), mx)
    torch.cuda.synchronize()
    if fused:
        bs = spec.block_size
        for i, s in enumerate(batch):
            b, o = slots[i] // bs, slots[i] % bs
            assert torch.equal(cache.k_cache[b, o].cpu().view(torch.int16), w.new_k[s].view(torch.int16))
            assert torch.equal(cache.v_cache[b, o].cpu().view(torch.int16), w.new_v[s].view(torch.int16))
    err = max_err(out.cpu(), oracle_out(w, batch))
    say(f"    groups {len(offs) - 1}, longest shared prefix {mx}: max abs err {err:.3e}")
    assert torch.isfinite(out.float()).all()
    assert err <= TOL[spec.dtype], err
