"""The host block pool under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The pool's sources (block_pool.cpp, status.cpp) are built with g++ and
``-fsanitize=address,undefined`` into a small line-protocol driver
(``tests/sanitize/pool_driver.cpp``), and the same random operation histories that the ABI
tests run through the library are run through the driver and compared, answer for answer and
state for state, with the oracle's block manager: allocate / extend (with copy-on-write) /
fork / free, moves between two pools, and prefix groups.  The pool is the block manager of the
111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解" §3.3
with the per-block reference counts of the gtnt.cn page "vLLM推理加速框架：PagedAttention与连续
批处理技术解析" §2.1.  Any sanitizer report ends the driver with a non-zero status and fails
the test that was running; the last test checks that the driver leaves cleanly (leak check
included).
"""

import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.block_manager import BlockManager
from paged_kv_cache_376_amd import binding as B
from tests.test_abi import _both_run, _move_both, _ops, _same_state, _swap_ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_376_amd", "csrc")
DRIVER_SRC = os.path.join(ROOT, "tests", "sanitize", "pool_driver.cpp")
_CODES = {name: code for code, name in B.STATUS_NAMES.items()}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


class _Driver:
    """The sanitized driver process: one command line in, one answer line out."""

    def __init__(self, exe):
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "halt_on_error=1:detect_leaks=1:abort_on_error=0"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        self.proc = subprocess.Popen([exe], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                     stderr=subprocess.PIPE, text=True, env=env)
        self.next_id = 0

    def ask(self, line):
        self.proc.stdin.write(line + "\n")
        self.proc.stdin.flush()
        ans = self.proc.stdout.readline()
        if not ans:
            err = self.proc.stderr.read()
            raise AssertionError(f"sanitized pool driver died on {line!r}:\n{err}")
        return ans.split()

    def close(self):
        self.proc.stdin.close()
        rc = self.proc.wait(timeout=60)
        return rc, self.proc.stderr.read()


def _ints(tok, tag, stop=None):
    """The integers after `tag` in an answer, up to the next tag (or `stop`)."""
    i = tok.index(tag) + 1
    out = []
    while i < len(tok) and (tok[i].lstrip("-").isdigit()):
        out.append(int(tok[i]))
        i += 1
    return out


class SanitizedPool:
    """The subset of binding.BlockPool's interface the ABI tests use, served by the driver."""

    def __init__(self, drv, num_blocks, block_size=16, free_order=None):
        self.d, self.id = drv, drv.next_id % 16
        drv.next_id += 1
        order = [] if free_order is None else [int(x) for x in free_order]
        self._check(self.d.ask(f"create {self.id} {num_blocks} {block_size} {len(order)} {' '.join(map(str, order))}"))
        self.block_size, self.num_blocks = block_size, num_blocks

    @staticmethod
    def _check(tok):
        if tok[0] != "PKV_OK":
            raise B.PkvError(_CODES.get(tok[0], -1), tok[0])
        return tok

    def close(self):
        self.d.ask(f"destroy {self.id}")

    def seq_allocate(self, seq, n):
        return _ints(self._check(self.d.ask(f"alloc {self.id} {seq} {n}")), "B")

    def seq_extend(self, seq, n):
        tok = self._check(self.d.ask(f"extend {self.id} {seq} {n}"))
        cow = _ints(tok, "C")
        return np.array(_ints(tok, "S"), dtype=np.int64), [tuple(cow)] if cow else []

    def seq_fork(self, parent, child):
        self._check(self.d.ask(f"fork {self.id} {parent} {child}"))

    def seq_free(self, seq):
        self._check(self.d.ask(f"free {self.id} {seq}"))

    def seq_context_len(self, seq):
        return int(self.d.ask(f"len {self.id} {seq}")[1])

    def free_list(self):
        return _ints(self.d.ask(f"freelist {self.id}"), "F")

    def ref_count(self, block):
        return _ints(self.d.ask(f"refs {self.id}"), "R")[block]

    def num_seqs(self):
        return int(self.d.ask(f"nseqs {self.id}")[1])

    def block_tables(self, seqs, maxb):
        seqs = [int(s) for s in seqs]
        tok = self._check(self.d.ask(f"tables {self.id} {maxb} {len(seqs)} {' '.join(map(str, seqs))}"))
        return np.array(_ints(tok, "T"), dtype=np.int32).reshape(len(seqs), maxb), np.array(_ints(tok, "L"))

    def move_seqs(self, dst, seqs):
        seqs = [int(s) for s in seqs]
        cap = sum(-(-max(self.seq_context_len(s), 0) // self.block_size) for s in seqs)
        tok = self._check(self.d.ask(f"move {self.id} {dst.id} {cap} {len(seqs)} {' '.join(map(str, seqs))}"))
        return np.array(_ints(tok, "P"), dtype=np.int32).reshape(-1, 2)

    def prefix_groups(self, seqs, min_prefix=0):
        seqs = [int(s) for s in seqs]
        tok = self._check(self.d.ask(f"groups {self.id} {min_prefix} {len(seqs)} {' '.join(map(str, seqs))}"))
        return (np.array(_ints(tok, "P"), dtype=np.int32), np.array(_ints(tok, "O"), dtype=np.int32),
                np.array(_ints(tok, "M"), dtype=np.int32), int(tok[tok.index("X") + 1]))


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("asan") / "pool_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", DRIVER_SRC, os.path.join(CSRC, "block_pool.cpp"),
           os.path.join(CSRC, "status.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    drv = _Driver(exe)
    yield drv
    if drv.proc.poll() is None:
        drv.close()


@settings(max_examples=150, deadline=None)
@given(ops=_ops, nb=st.integers(1, 24), bs=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 1000))
def test_sanitized_pool_matches_oracle_on_random_histories(driver, ops, nb, bs, seed):
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = SanitizedPool(driver, nb, bs, order)
    bm = BlockManager(nb, bs, order.tolist())
    for op in ops:
        _both_run(pool, bm, op)
        _same_state(pool, bm)
    pool.close()


@settings(max_examples=100, deadline=None)
@given(ops=_swap_ops, nb=st.integers(1, 20), nh=st.integers(1, 20), bs=st.sampled_from([1, 4, 16]),
       seed=st.integers(0, 1000))
def test_sanitized_move_seqs_matches_oracle(driver, ops, nb, nh, bs, seed):
    rng = np.random.default_rng(seed)
    o1, o2 = rng.permutation(nb).astype(np.int32), rng.permutation(nh).astype(np.int32)
    pools = [SanitizedPool(driver, nb, bs, o1), SanitizedPool(driver, nh, bs, o2)]
    bms = [BlockManager(nb, bs, o1.tolist()), BlockManager(nh, bs, o2.tolist())]
    for kind, a, b, n, seqs, side in ops:
        if kind == "move":
            _move_both(pools, bms, side, seqs)
        else:
            _both_run(pools[side], bms[side], (kind, a, b, n))
        _same_state(pools[0], bms[0])
        _same_state(pools[1], bms[1])
    for p in pools:
        p.close()


@settings(max_examples=100, deadline=None)
@given(ops=_ops, nb=st.integers(1, 40), bs=st.sampled_from([1, 4, 8, 16, 32]), seed=st.integers(0, 1000),
       min_prefix=st.sampled_from([0, 16, 48]))
def test_sanitized_prefix_groups_match_oracle(driver, ops, nb, bs, seed, min_prefix):
    order = np.random.default_rng(seed).permutation(nb).astype(np.int32)
    pool = SanitizedPool(driver, nb, bs, order)
    bm = BlockManager(nb, bs, order.tolist())
    for op in ops:
        _both_run(pool, bm, op)
    batch = sorted(bm.block_tables)
    if len(batch) > 1:
        batch = batch + batch[:1]
    sp, offs, mem, mx = pool.prefix_groups(batch, min_prefix)
    esp, egroups = bm.prefix_groups(batch, min_prefix)
    assert sp.tolist() == esp
    assert [mem[offs[i]:offs[i + 1]].tolist() for i in range(len(offs) - 1)] == egroups
    assert mx == max(esp, default=0)
    pool.close()


def test_sanitized_pool_rejects_bad_arguments(driver):
    """Arguments the pool must refuse without touching memory: bad sizes and free orders,
    unknown sequences, negative counts, too small output buffers."""
    assert driver.ask("create 15 0 16 0")[0] == "PKV_ERR_INVALID_ARGUMENT"
    assert driver.ask("create 15 4 0 0")[0] == "PKV_ERR_INVALID_ARGUMENT"
    assert driver.ask("create 15 4 16 4 0 1 1 3")[0] == "PKV_ERR_INVALID_ARGUMENT"  # not a permutation
    assert driver.ask("create 15 4 16 4 0 1 2 9")[0] == "PKV_ERR_INVALID_ARGUMENT"  # id out of range
    assert driver.ask("create 15 4 16 0")[0] == "PKV_OK"
    assert driver.ask("alloc 15 1 -3")[0] == "PKV_ERR_INVALID_ARGUMENT"
    assert driver.ask("alloc 15 1 65")[0] == "PKV_ERR_OUT_OF_BLOCKS"
    assert driver.ask("extend 15 7 1")[0] == "PKV_ERR_NOT_FOUND"
    assert driver.ask("alloc 15 1 40")[0] == "PKV_OK"
    assert driver.ask("tables 15 2 1 1")[0] == "PKV_ERR_INVALID_ARGUMENT"  # table of 3 blocks
    assert driver.ask("tables 15 3 1 9")[0] == "PKV_ERR_NOT_FOUND"
    assert driver.ask("move 15 15 4 1 1")[0] == "PKV_ERR_INVALID_ARGUMENT"  # same pool
    assert driver.ask("groups 15 -1 1 1")[0] == "PKV_ERR_INVALID_ARGUMENT"
    assert driver.ask("groups 15 0 1 9")[0] == "PKV_ERR_NOT_FOUND"
    assert driver.ask("destroy 15")[0] == "PKV_OK"


def test_sanitized_driver_exits_cleanly(driver):
    """Last: every pool destroyed at end of input, no leak, no sanitizer report."""
    rc, err = driver.close()
    assert rc == 0 and "Sanitizer" not in err and "runtime error" not in err, err
