"""Benchmark of one decode step of one layer: KV append + paged decode attention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config gqa_bf16] [--partition 0]

A step is the whole hot path over one batch: the append of one new token per sequence
(``pkv_kv_cache_append``) followed by paged decode attention over every context including
that token (``pkv_paged_attn_decode``), with all inputs resident in HBM.  The default
workload is the Llama-3-70B-shaped GQA decode (batch 256, 64 query / 8 KV heads, head dim
128, bf16, lognormal context lengths with median 512 clipped to [16, 8192], seed 0).

Prints one JSON line: KV GB/s of the step (bytes of K and V the decode reads per step over
the step time), the fraction of MI355X's 8 TB/s HBM peak, attention-only decode tokens/s
at the 80-layer 70B shape, a roofline record for the decode launch (timed with HIP events
on its stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
LAYERS_70B = 80        # layers of the 70B model whose shape the default workload has


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(w):
    """Bytes one decode must move: every context's K and V rows read once, q read, out
    written, block-table entries and context lengths read.  Scratch traffic of split
    sequences is an artefact of how the work is cut and is not counted (so the achieved
    rate is a lower bound).  Returns (kv_bytes, decode_bytes)."""
    sp = w.spec
    e = {"float32": 4, "float16": 2, "bfloat16": 2}[sp.dtype]
    lens = [int(L) + 1 for L in w.context_lens]
    kv = sum(lens) * sp.num_kv_heads * sp.head_dim * 2 * e
    qo = 2 * sp.num_seqs * sp.num_q_heads * sp.head_dim * e
    tables = 4 * sum(-(-L // 16) for L in lens) + 4 * sp.num_seqs
    return kv, kv + qo + tables


def prefix_shared_bytes(w, seq_prefix, group_offsets, group_members):
    """Bytes the prefix-shared decode must move: each group's shared prefix K/V read once per
    group, every sequence's own remainder (with its appended token) once, q read, out written,
    block-table entries and context lengths read.  Partial results of the prefix / suffix split
    are not counted, as for the plain decode.  Returns (kv_bytes_read, decode_bytes)."""
    sp = w.spec
    e = {"float32": 4, "float16": 2, "bfloat16": 2}[sp.dtype]
    lens = [int(L) + 1 for L in w.context_lens]
    tokens = sum(lens) - sum(int(p) for p in seq_prefix)
    tokens += sum(int(seq_prefix[group_members[group_offsets[g]]]) for g in range(len(group_offsets) - 1))
    kv = tokens * sp.num_kv_heads * sp.head_dim * 2 * e
    qo = 2 * sp.num_seqs * sp.num_q_heads * sp.head_dim * e
    tables = 4 * sum(-(-L // 16) for L in lens) + 4 * sp.num_seqs
    return kv, kv + qo + tables


# rocprofv3 counter summaries (FETCH_SIZE / WRITE_SIZE, calibrated on a copy of known size) of the
# decode call of each workload, keyed by (workload, mode), and the kernel sources they were taken on
_CSRC = os.path.join(ROOT, "paged_kv_cache_376_amd", "csrc")
SK_SOURCES = [os.path.join(_CSRC, f) for f in ("paged_attn_sk.hip", "tile_common.h", "stream_k.h", "dtypes.h")]
PREFIX_SOURCES = SK_SOURCES + [os.path.join(_CSRC, f) for f in ("paged_attn_prefix.hip", "prefix.h", "prefix_body.h")]
FIXED_SOURCES = [os.path.join(_CSRC, f) for f in ("paged_attn.hip", "dtypes.h")]
COUNTER_FILES = {
    ("gqa_bf16", "fused"): ("decode_gqa_bf16_B256_counters.md", SK_SOURCES),
    ("mha_fp16", "fused"): ("decode_mha_fp16_B64_counters.md", SK_SOURCES),
    ("long_bf16", "fused"): ("decode_long_bf16_B8_counters.md", SK_SOURCES),
    ("prefix_bf16", "fused"): ("decode_prefix_bf16_B128_counters.md", SK_SOURCES),
    ("tiny_fp32", "fused"): ("decode_tiny_fp32_B4_counters.md", FIXED_SOURCES),
    ("prefix_bf16", "prefix"): ("decode_prefix_bf16_B128_shared_counters.md", PREFIX_SOURCES),
}


def source_sha256(files=None):
    """SHA-256 of kernel sources with comments and whitespace removed: an edit of a comment does
    not change what the counters measured, an edit of code does."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in files or SK_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def counter_traffic(config="gqa_bf16", mode="fused"):
    """Calibrated HBM bytes of one decode call of this workload from its committed rocprofv3
    counter summary, or None when there is none or the kernel sources have changed since."""
    import re

    entry = COUNTER_FILES.get((config, mode))
    if entry is None:
        return None
    try:
        text = open(os.path.join(ROOT, "profiles", entry[0]), encoding="utf-8").read()
        want = re.search(r"kernel_source_sha256: ([0-9a-f]{64})", text).group(1)
        value = int(re.search(r"traffic_bytes_per_call: (\d+)", text).group(1))
        have = source_sha256(entry[1])
    except (OSError, AttributeError):
        return None
    return value if have == want else None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle on the host cores over a bounded sample of the same workload: the first
    sequences, as many as one pass of about budget_s / 3 seconds covers, timed three times
    (median reported), then three times more on one thread over the same sample."""
    import numpy as np
    import torch

    import oracle

    sp = w.spec
    e = {"float32": 4, "float16": 2, "bfloat16": 2}[sp.dtype]
    kv = {}

    def seq_kv(s):
        if s not in kv:
            kv[s] = w.seq_kv_after_append(s)
        return kv[s]

    def one_pass(seqs):
        nbytes, t = 0, 0.0
        for s in seqs:
            k, v = seq_kv(s)
            t0 = time.perf_counter()
            oracle.decode_attention(w.q[s:s + 1], [k], [v], w.scale)
            t += time.perf_counter() - t0
            nbytes += k.shape[0] * sp.num_kv_heads * sp.head_dim * 2 * e
        return nbytes, t

    one_pass([0])  # warm-up
    # the sample: sequences in order until one pass has taken budget_s / 3
    sample, t_first, nbytes = [], 0.0, 0
    for s in range(sp.num_seqs):
        b_s, t_s = one_pass([s])
        sample.append(s)
        t_first += t_s
        nbytes += b_s
        if t_first >= budget_s / 3:
            break
    runs = [nbytes / t_first / 1e9] + [nbytes / one_pass(sample)[1] / 1e9 for _ in range(2)]
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        blas = [f"{i.get('internal_api')}:{i.get('num_threads')}" for i in threadpool_info()]
    except Exception:  # pragma: no cover - informational only
        blas, threadpool_limits = [], None
    cores = max([torch.get_num_threads()] + [int(b.split(":")[1]) for b in blas if b.split(":")[1].isdigit()])
    # one thread: BLAS pools and torch limited to 1
    single = None
    small = sample
    n_threads = torch.get_num_threads()
    try:
        torch.set_num_threads(1)
        passes = []
        for _ in range(3):
            if threadpool_limits is not None:
                with threadpool_limits(limits=1):
                    passes.append(one_pass(small))
            else:
                passes.append(one_pass(small))
        b1 = passes[0][0]
        t1 = float(np.median([t for _, t in passes]))
        single = {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "runs": [round(b / t / 1e9, 4) for b, t in passes],
                  "sample": f"the same {len(small)} sequences ({b1 / 1e6:.1f} MB of K/V, median of 3 passes "
                            f"of {t1:.1f} s)"}
    finally:
        torch.set_num_threads(n_threads)
    all_cores = {"value": round(float(np.median(runs)), 4), "unit": "GB/s", "cores": cores,
                 "runs": [round(r, 4) for r in runs],
                 "threads": f"torch {n_threads}, {', '.join(blas) or 'blas n/a'}"}
    # the faster of the two configurations is the baseline (its per-sequence products are small
    # enough that threaded BLAS can lose to one thread)
    best = single if single is not None and single["value"] > all_cores["value"] else all_cores
    return {"value": best["value"], "unit": "GB/s", "cores": best["cores"],
            "kind": "oracle",
            "sample": f"first {len(sample)} of {sp.num_seqs} sequences of the same workload "
                      f"({nbytes / 1e6:.1f} MB of K/V per pass), fp64 numpy, upcast inside the timer; "
                      f"all cores: median of 3 timed passes after a warm-up; one thread: median of 3 passes; the "
                      f"faster is reported; host cores available {len(os.sched_getaffinity(0))}",
            "all_cores": all_cores,
            "single_thread": single,
            "cpu_model": _cpu_model(),
            "note": "the oracle is a correctness tool, not a tuned CPU kernel"}


# Block shape of the default workload's pools: 16 tokens x 8 KV heads x 128 x bf16 = 32 KiB.
BLOCK_SHAPE = (16, 8, 128)
PCIE_PEAK_GBS = 64.0  # host link of an MI355X: PCIe 5.0 x16, per direction, vendor figure


def _time_calls(fn, steps, warmup, stream):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps / 1e3  # seconds per call


def read_ceiling(dev):
    """The device's practical HBM read ceiling: a plain contiguous read of 1 GiB (16-byte
    loads, 8 in flight per thread, 2048 work-groups) by the probe library the build makes
    next to libpagedkv, timed with HIP events on the launch stream.  None when the probe
    library is missing."""
    import ctypes

    import torch

    from paged_kv_cache_376_amd import build as pkv_build

    if not os.path.exists(pkv_build.PROBE_PATH):
        return None
    probe = ctypes.CDLL(pkv_build.PROBE_PATH)
    fn = probe.pkv_read_ceiling_pass
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = 1 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(2048, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def one():
        rc = fn(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"read-ceiling probe launch failed ({rc})")

    t = _time_calls(one, 20, 3, stream)
    del buf
    gbs = nbytes / t / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "probe": "contiguous read of 1 GiB, 16-byte loads, 8 in flight per thread, 2048 work-groups of 256"}


def bench_copy_blocks(args, dev):
    """pkv_copy_blocks on the default workload's block shape: 4096 (source, destination)
    pairs drawn from a 16384-block pool per call; bytes = pairs x 2 pools x block x (read +
    write)."""
    import numpy as np
    import torch

    from paged_kv_cache_376_amd import binding

    nb, n = 16384, 4096
    rng = np.random.default_rng(args.seed)
    k = torch.randn((nb,) + BLOCK_SHAPE, dtype=torch.bfloat16, device=dev)
    v = torch.randn((nb,) + BLOCK_SHAPE, dtype=torch.bfloat16, device=dev)
    perm = rng.permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    block_bytes = int(np.prod(BLOCK_SHAPE)) * 2
    moved = n * 2 * block_bytes * 2
    t = _time_calls(lambda: binding.copy_blocks(k, v, pairs, stream=stream), args.steps, args.warmup, stream)
    gbs = moved / t / 1e9
    log(f"copy_blocks: {n} pairs of {block_bytes} B blocks per pool, {t * 1e6:.1f} us per call, {gbs:.0f} GB/s")
    return {"metric": "pkv_copy_blocks (copy-on-write) GB/s, read + write", "value": round(gbs, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (copied as bytes)",
            "data": "synthetic random pools and pairs",
            "config": {"workload": f"copy_blocks: {n} pairs from a {nb}-block pool, block {BLOCK_SHAPE} bf16",
                       "bytes_per_call": moved},
            "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm", "achieved": round(gbs, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": None, "bytes_per_launch": moved, "avg_launch_us": round(t * 1e6, 2)}}


def bench_swap(args, dev):
    """pkv_swap_blocks between a device pool and a pinned host pool of the default block shape:
    2048 blocks out (device -> host) and 2048 back in per call; against one copy command per
    block (what a runtime memcpy per block costs)."""
    import numpy as np
    import torch

    from paged_kv_cache_376_amd import binding

    nb, nh, n = 8192, 4096, 2048
    rng = np.random.default_rng(args.seed)
    k = torch.randn((nb,) + BLOCK_SHAPE, dtype=torch.bfloat16, device=dev)
    v = torch.randn((nb,) + BLOCK_SHAPE, dtype=torch.bfloat16, device=dev)
    hk = torch.empty((nh,) + BLOCK_SHAPE, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((nh,) + BLOCK_SHAPE, dtype=torch.bfloat16).pin_memory()
    dev_ids = rng.permutation(nb)[:n]
    host_ids = rng.permutation(nh)[:n]
    out_pairs = torch.from_numpy(np.stack([dev_ids, host_ids], axis=1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([host_ids, dev_ids], axis=1).astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    block_bytes = int(np.prod(BLOCK_SHAPE)) * 2
    moved = n * 2 * block_bytes  # bytes over the link per direction per call
    steps = max(3, args.steps // 5)
    t_out = _time_calls(lambda: binding.swap_blocks(hk, hv, k, v, out_pairs, stream=stream), steps, 2, stream)
    t_in = _time_calls(lambda: binding.swap_blocks(k, v, hk, hv, in_pairs, stream=stream), steps, 2, stream)
    ids_d, ids_h = dev_ids.tolist(), host_ids.tolist()

    def per_block_out():
        for a, b in zip(ids_d, ids_h):
            hk[b].copy_(k[a], non_blocking=True)
            hv[b].copy_(v[a], non_blocking=True)

    t_ref = _time_calls(per_block_out, 2, 1, stream)
    g_out, g_in, g_ref = moved / t_out / 1e9, moved / t_in / 1e9, moved / t_ref / 1e9
    log(f"swap: {n} blocks x 2 pools ({moved / 1e6:.0f} MB) out {t_out * 1e3:.2f} ms ({g_out:.1f} GB/s), "
        f"in {t_in * 1e3:.2f} ms ({g_in:.1f} GB/s); one copy command per block: {t_ref * 1e3:.2f} ms ({g_ref:.1f} GB/s)")
    return {"metric": "pkv_swap_blocks device<->pinned host GB/s (out, in)", "value": round(min(g_out, g_in), 2),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": 2,
            "ms_per_step": round((t_out + t_in) * 1e3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16 (copied as bytes)", "data": "synthetic random pools and pairs",
            "swap_out_gbs": round(g_out, 2), "swap_in_gbs": round(g_in, 2),
            "per_block_copy_commands_out_gbs": round(g_ref, 2),
            "config": {"workload": f"swap: {n} blocks of {BLOCK_SHAPE} bf16 per pool, K and V, device pool {nb} "
                                   f"blocks, pinned host pool {nh} blocks", "bytes_per_call": moved},
            "roofline": {"kernel": "copy_blocks_kernel (host side pinned)", "bound": "pcie",
                         "achieved": round(min(g_out, g_in), 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                         "frac": round(min(g_out, g_in) / PCIE_PEAK_GBS, 4), "traffic": None,
                         "bytes_per_launch": moved, "avg_launch_us": round((t_out + t_in) / 2 * 1e6, 2)}}


def bench_append(args, dev):
    """pkv_kv_cache_append of a prefill chunk (multi-token append through the same scatter) into
    the default workload's pools: T tokens of 8 KV heads x 128 bf16 to the slots of fresh
    sequences of 1024 tokens taken from the host pool; bytes = T rows x 2 (K, V) x (read +
    write)."""
    import numpy as np
    import torch

    from paged_kv_cache_376_amd import binding
    from paged_kv_cache_376_amd.cache import PagedKVCache

    T = args.append_tokens
    bs = args.block_size or 16
    hkv, d = BLOCK_SHAPE[1], BLOCK_SHAPE[2]
    nb = -(-T // bs) + 64
    rng = np.random.default_rng(args.seed)
    cache = PagedKVCache(nb, hkv, d, torch.bfloat16, dev, free_order=rng.permutation(nb).astype(np.int32),
                         block_size=bs)
    slots = []
    for s in range(-(-T // 1024)):
        n = min(1024, T - 1024 * s)
        cache.pool.seq_allocate(s, 0)
        sl, _ = cache.pool.seq_extend(s, n)
        slots.append(sl)
    slot_t = torch.from_numpy(np.concatenate(slots)).to(dev)
    key = torch.randn((T, hkv, d), dtype=torch.bfloat16, device=dev)
    value = torch.randn((T, hkv, d), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    moved = T * hkv * d * 2 * 2 * 2
    t = _time_calls(lambda: binding.kv_cache_append(key, value, cache.k_cache, cache.v_cache, slot_t, stream=stream),
                    args.steps, args.warmup, stream)
    gbs = moved / t / 1e9
    log(f"append: {T} tokens ({hkv}x{d} bf16 per token and pool, block {bs}), {t * 1e6:.1f} us per call, {gbs:.0f} GB/s")
    return {"metric": "pkv_kv_cache_append (prefill chunk) GB/s, read + write", "value": round(gbs, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (copied as bytes)",
            "data": "synthetic rows, slots of fresh 1024-token sequences",
            "config": {"workload": f"append: {T} tokens, Hkv {hkv}, D {d}, bf16, block {bs}", "bytes_per_call": moved},
            "roofline": {"kernel": "kv_append_kernel", "bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "bytes_per_launch": moved, "avg_launch_us": round(t * 1e6, 2)}}


def fused_append_bytes(w):
    """Bytes the fused call moves for its append beyond the decode's own: each sequence's new K
    and V rows are read as part of its context (counted in the K/V bytes) and written once to
    their pool slots."""
    sp = w.spec
    e = {"float32": 4, "float16": 2, "bfloat16": 2}[sp.dtype]
    return 2 * sp.num_seqs * sp.num_kv_heads * sp.head_dim * e


def append_call_bytes(w):
    """Bytes of the append as a call of its own (pkv_kv_cache_append): the new K and V rows read
    from the input and written to the pools, and the 8-byte slots."""
    return 2 * fused_append_bytes(w) + 8 * w.spec.num_seqs


def measure_step(w, dev, steps, warmup, partition=0, mode="fused"):
    """Builds the workload's pools, lets the host pool take each sequence's next slot, and times
    the decode step of `mode`:
      fused    one pkv_paged_attn_decode_append call (the default step);
      separate pkv_kv_cache_append, then pkv_paged_attn_decode;
      prefix   one pkv_paged_attn_decode_prefix_append call (groups from the pool).
    K steps run back to back between two HIP events on the launch stream (after W warm-up
    steps); a second pass of K steps puts events around every call for the per-call times.  The
    append call is also timed on its own.  Returns the times and the byte counts."""
    import numpy as np
    import torch

    from paged_kv_cache_376_amd import binding
    from paged_kv_cache_376_amd.cache import build_cache

    sp = w.spec
    t0 = time.perf_counter()
    cache = build_cache(w, dev)
    torch.cuda.synchronize()
    log(f"{sp.name}: pool built in {time.perf_counter() - t0:.1f} s ({w.num_blocks} blocks)")
    seqs = list(range(sp.num_seqs))
    # Host side of the step, done once: every sequence takes the slot of its next token.
    slots = np.zeros(sp.num_seqs, dtype=np.int64)
    for i, s in enumerate(seqs):
        sl, cow = cache.pool.seq_extend(s, 1)
        cache.copy_blocks(cow)
        slots[i] = sl[0]
    slot_t = torch.from_numpy(slots).to(dev)
    new_k = w.new_k.to(dev).contiguous()
    new_v = w.new_v.to(dev).contiguous()
    bt, ctx, maxc = cache.tables(seqs)
    q = w.q.to(dev).contiguous()
    out = torch.empty_like(q)
    part = binding.paged_attn_partition_size(sp.num_seqs, sp.num_q_heads, sp.num_kv_heads,
                                             sp.head_dim, maxc, partition, sp.dtype)
    ws_bytes = binding.paged_attn_workspace_bytes(sp.num_seqs, sp.num_q_heads, sp.num_kv_heads,
                                                  sp.head_dim, maxc, partition, sp.dtype)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def append_call():
        binding.kv_cache_append(new_k, new_v, cache.k_cache, cache.v_cache, slot_t, stream=stream)

    def decode_call():
        binding.paged_attn_decode(out, q, cache.k_cache, cache.v_cache, bt, ctx, maxc, w.scale,
                                  workspace=ws, partition_size=partition, stream=stream)

    def fused_call():
        binding.paged_attn_decode_append(out, q, new_k, new_v, cache.k_cache, cache.v_cache, bt, ctx,
                                         maxc, w.scale, workspace=ws, partition_size=partition,
                                         stream=stream)

    groups = None
    if mode == "prefix":
        sp_, offs_, mem_, mx_ = cache.pool.prefix_groups(seqs)
        groups = (sp_, offs_, mem_, mx_)
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        sp_d, offs_d, mem_d = to_dev(sp_), to_dev(offs_), to_dev(mem_)
        pws = binding.paged_attn_decode_prefix_workspace_bytes(sp.num_seqs, sp.num_q_heads, sp.num_kv_heads,
                                                               sp.head_dim, maxc, mx_, sp.dtype)
        pws_t = torch.empty(max(pws, 16), dtype=torch.uint8, device=dev)
        log(f"prefix groups: {len(offs_) - 1}, longest shared prefix {mx_} tokens")

        def prefix_call():
            binding.paged_attn_decode_prefix_append(out, q, new_k, new_v, cache.k_cache, cache.v_cache, bt, ctx, maxc,
                                                    w.scale, sp_d, offs_d, mem_d, mx_, workspace=pws_t,
                                                    stream=stream)

    calls = {"prefix": lambda: [prefix_call], "separate": lambda: [append_call, decode_call],
             "fused": lambda: [fused_call]}[mode]()
    log(f"{sp.name}: warmup {warmup} steps ({mode}, partition {part or 'even split'}, workspace {ws_bytes} B)")
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()

    # Timed region: K steps back to back, bracketed by synchronize + events on the launch stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        for c in calls:
            c()
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    # Per-call durations for the roofline record: a second pass of K steps with HIP events on
    # the launch stream around every call (kept out of the step timing above).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    t_calls = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(calls))] for i in range(steps)])
    t_dec = t_calls[:, -1]
    t_app = t_calls[:, 0] if mode == "separate" else None
    # the append alone, back to back (it rewrites the same rows into the same slots)
    append_us = _time_calls(append_call, steps, warmup, stream) * 1e6
    if mode != "separate":
        log(f"{sp.name}: step {ms_step * 1e3:.1f} us: fused append+decode call median {np.median(t_dec) * 1e3:.1f} "
            f"us (p10 {np.percentile(t_dec, 10) * 1e3:.1f}, p90 {np.percentile(t_dec, 90) * 1e3:.1f}); "
            f"append alone {append_us:.1f} us")
    else:
        log(f"{sp.name}: step {ms_step * 1e3:.1f} us: append {t_app.mean() * 1e3:.1f} us, decode "
            f"median {np.median(t_dec) * 1e3:.1f} us (p10 {np.percentile(t_dec, 10) * 1e3:.1f}, "
            f"p90 {np.percentile(t_dec, 90) * 1e3:.1f})")

    kv_bytes, dec_bytes = algorithmic_bytes(w)
    kv_read = kv_bytes
    if mode == "prefix":
        # the method reads each shared prefix once per group: that is the roofline's byte count
        kv_read, dec_bytes = prefix_shared_bytes(w, *groups[:3])
    if mode != "separate":
        dec_bytes += fused_append_bytes(w)
    del cache, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "t_dec": t_dec, "t_app": t_app, "append_us": append_us, "part": part,
            "ws_bytes": ws_bytes, "kv_bytes": kv_bytes, "kv_read": kv_read, "dec_bytes": dec_bytes,
            "groups": groups}


def _config_record(w, m, mode):
    """One per_config entry from measure_step's result."""
    import numpy as np

    dec_s = float(m["t_dec"].mean()) / 1e3
    step_s = m["ms_step"] / 1e3
    achieved = m["dec_bytes"] / dec_s / 1e9
    sp = w.spec
    rec = {
        "workload": f"{sp.name}: B={sp.num_seqs}, Hq={sp.num_q_heads}, Hkv={sp.num_kv_heads}, D={sp.head_dim}, "
                    f"{sp.dtype}, block {sp.block_size}, lengths {sp.lengths}, +1 appended token per sequence",
        "step_calls": {"fused": "pkv_paged_attn_decode_append",
                       "separate": "pkv_kv_cache_append + pkv_paged_attn_decode",
                       "prefix": "pkv_paged_attn_decode_prefix_append (append fused into the decode)"}[mode],
        "step_us": round(m["ms_step"] * 1e3, 2),
        "kv_bytes_per_step": m["kv_bytes"],
        "kv_gbs": round(m["kv_bytes"] / step_s / 1e9, 2),
        "pct_hbm_peak": round(100.0 * m["kv_read"] / step_s / 1e9 / HBM_PEAK_GBS, 2),
        "decode_us_median": round(float(np.median(m["t_dec"])) * 1e3, 2),
        "decode_roofline_frac": round(achieved / HBM_PEAK_GBS, 4),
        "decode_bytes_per_launch": m["dec_bytes"],
        "decode_traffic_per_launch": counter_traffic(sp.name, mode),
        "append_us": round(m["append_us"], 2),
        "decode_tokens_per_s_per_layer": round(sp.num_seqs / step_s, 1),
        "partition_tokens": m["part"] if m["part"] else "even split over the GPU",
    }
    if mode == "prefix":
        rec["kv_bytes_read_per_step"] = m["kv_read"]
        rec["note"] = ("pct_hbm_peak and the roofline count each group's shared prefix once; kv_gbs counts every "
                       "sequence's whole context")
    if sp.name == "tiny_fp32":
        rec["note"] = "latency-bound (309 KB of K/V); a correctness case"
    return rec


def per_config_records(w_head, head, dev, args):
    """Every workload the benchmark knows, timed the same way as the headline step (fused call,
    seed args.seed): the headline's own numbers for gqa_bf16, and for prefix_bf16 also the
    prefix-shared call."""
    from paged_kv_cache_376_amd import workloads

    recs = {"gqa_bf16": {
        "workload": head["config"]["workload"], "step_calls": "pkv_paged_attn_decode_append",
        "step_us": round(head["ms_per_step"] * 1e3, 2), "kv_bytes_per_step": head["config"]["kv_bytes_per_step"],
        "kv_gbs": head["value"], "pct_hbm_peak": head["pct_hbm_peak"], "decode_us_median": head["decode_us_median"],
        "decode_roofline_frac": head["roofline"]["frac"], "decode_bytes_per_launch": head["roofline"]["bytes_per_launch"],
        "decode_traffic_per_launch": head["roofline"]["traffic"],
        "append_us": head["append_us"], "decode_tokens_per_s_per_layer": head["decode_tokens_per_s_per_layer"],
        "partition_tokens": head["config"]["partition_tokens"]}}
    for name, mode in (("tiny_fp32", "fused"), ("mha_fp16", "fused"), ("long_bf16", "fused"),
                       ("prefix_bf16", "fused"), ("prefix_bf16", "prefix")):
        w = workloads.make_workload(name, args.seed)
        m = measure_step(w, dev, args.steps, args.warmup, 0, mode)
        recs[name if mode == "fused" else name + "_shared"] = _config_record(w, m, mode)
    return recs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gqa_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--separate", action="store_true",
                    help="time the step as two calls (pkv_kv_cache_append, then "
                         "pkv_paged_attn_decode) instead of one pkv_paged_attn_decode_append")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per_config record (the other workloads, each timed the same way)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--op", choices=["step", "copy_blocks", "swap", "append"], default="step",
                    help="step: the decode step (default); copy_blocks: pkv_copy_blocks "
                         "(copy-on-write) GB/s; swap: pkv_swap_blocks device<->pinned host GB/s; "
                         "append: pkv_kv_cache_append of a prefill chunk GB/s")
    ap.add_argument("--prefix-shared", action="store_true",
                    help="decode with pkv_paged_attn_decode_prefix_append (groups from "
                         "pkv_pool_prefix_groups, append fused)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="tokens per pool block (default: the workload's, 16)")
    ap.add_argument("--append-tokens", type=int, default=16384,
                    help="tokens of the prefill chunk for --op append")
    args = ap.parse_args()

    if args.gpus != 1:
        sys.exit("bench.py measures one GPU only: the library has no multi-GPU path "
                 "(decode attention shards by KV head or sequence with no exchange; see the "
                 "design notes). Run with --gpus 1.")

    import numpy as np
    import torch

    from paged_kv_cache_376_amd import binding, workloads

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a HIP device")
    binding.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.op != "step":
        result = {"copy_blocks": bench_copy_blocks, "swap": bench_swap, "append": bench_append}[args.op](args, dev)
        print(json.dumps(result), flush=True)
        return

    log(f"generating workload {args.config} seed {args.seed}")
    w = workloads.make_workload(args.config, args.seed,
                                **({"block_size": args.block_size} if args.block_size else {}))
    sp = w.spec
    mode = "prefix" if args.prefix_shared else "separate" if args.separate else "fused"
    m = measure_step(w, dev, args.steps, args.warmup, args.partition, mode)
    ms_step, t_dec, t_app, part = m["ms_step"], m["t_dec"], m["t_app"], m["part"]
    kv_bytes, kv_read, dec_bytes = m["kv_bytes"], m["kv_read"], m["dec_bytes"]
    dec_s = float(t_dec.mean()) / 1e3
    gbs = kv_bytes / (ms_step / 1e3) / 1e9
    achieved = dec_bytes / dec_s / 1e9
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copy done")

    result = {
        "metric": "paged decode attention KV GB/s and % HBM peak; tokens/s at 70B-GQA shape",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "float16": "f16", "bfloat16": "bf16"}[sp.dtype],
        "data": "synthetic (seeded N(0,1) K/V/q, shuffled physical blocks)",
        # K/V bytes actually read per step over the step time (differs from `value` only when
        # prefixes are shared: `value` then counts every sequence's whole context)
        "pct_hbm_peak": round(100.0 * kv_read / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s_per_layer": round(sp.num_seqs / (ms_step / 1e3), 1),
        "decode_tokens_per_s_70b_shape_attention_only": round(sp.num_seqs / (LAYERS_70B * ms_step / 1e3), 1),
        # pkv_kv_cache_append of the step's new rows, timed on its own (the fused call does the
        # same writes inside the decode): mean time per call and its algorithmic bytes (new rows
        # read and written, 8-byte slots) over that time
        "append_us": round(m["append_us"], 2),
        "append_gbs": round(append_call_bytes(w) / (m["append_us"] / 1e6) / 1e9, 2),
        "decode_us_median": round(float(np.median(t_dec)) * 1e3, 2),
        "decode_us_p10": round(float(np.percentile(t_dec, 10)) * 1e3, 2),
        "decode_us_p90": round(float(np.percentile(t_dec, 90)) * 1e3, 2),
        "step_calls": "pkv_paged_attn_decode_prefix_append (append fused into the decode)" if args.prefix_shared
                      else "pkv_kv_cache_append + pkv_paged_attn_decode" if args.separate
                      else "pkv_paged_attn_decode_append (append fused into the decode)",
        "config": {
            "workload": f"{sp.name}: paged decode, B={sp.num_seqs}, Hq={sp.num_q_heads}, "
                        f"Hkv={sp.num_kv_heads}, D={sp.head_dim}, block {sp.block_size}, {sp.dtype}, "
                        f"lengths {sp.lengths}, seed {args.seed}, +1 appended token per sequence",
            "num_seqs": sp.num_seqs,
            "kv_tokens": int(w.context_lens.sum()) + sp.num_seqs,
            "kv_bytes_per_step": kv_bytes,
            "kv_bytes_read_per_step": kv_read,
            "partition_tokens": part if part else "even split over the GPU",
            "pool_blocks": w.num_blocks,
        },
        "roofline": {
            "kernel": ("pkv_paged_attn_decode_prefix_append" if args.prefix_shared else
                       "pkv_paged_attn_decode" if args.separate else "pkv_paged_attn_decode_append") +
                      (" (prefix pass and suffix decode in one launch, then the finalize kernel, which "
                       "also writes the new rows)"
                       if args.prefix_shared else
                       f" (fixed partitions of {part} tokens: decode kernel, then a reduce when a "
                       f"sequence spans several)" if part else
                       " (decode kernel + merge of sequences cut by the split)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            # counters are taken per workload (seed 0, default block size and split)
            "traffic": counter_traffic(args.config, mode) if (args.seed == 0 and args.partition == 0
                                                              and not args.block_size) else None,
            "bytes_per_launch": dec_bytes,
            "avg_launch_us": round(dec_s * 1e6, 2),
        },
    }
    ceiling = read_ceiling(dev)
    if ceiling is not None:
        log(f"practical read ceiling of this device: {ceiling['value']:.0f} GB/s "
            f"({100 * ceiling['frac_of_peak']:.1f}% of {HBM_PEAK_GBS:.0f})")
        result["read_ceiling"] = ceiling
        result["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["value"], 4)
    if not args.no_per_config and args.config == "gqa_bf16" and mode == "fused" and not args.block_size \
            and args.partition == 0:
        del m
        result["per_config"] = per_config_records(w, result, dev, args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        result["cpu_baseline"]["gpu_speedup"] = round(gbs / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
