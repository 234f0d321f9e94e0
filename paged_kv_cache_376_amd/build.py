"""Builds libpagedkv.so (and the benchmark's read-ceiling probe) in-tree with hipcc for gfx950.

Every call compiles from scratch (objects under ``_build/`` at the repo root, the shared
library next to this file).  ``python -m paged_kv_cache_376_amd.build`` does the same.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpagedkv.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

HOST_SOURCES = ["status.cpp", "block_pool.cpp"]
DEVICE_SOURCES = ["kv_append.hip", "paged_attn.hip", "paged_attn_sk.hip", "block_copy.hip", "paged_attn_prefix.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]
# Packed-fp32 VALU ops are kept out of the generated code on purpose.
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def _compile(src: str, verbose: bool) -> str:
    hipcc = _hipcc()
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc, *DEVICE_FLAGS, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [hipcc, "-x", "c++", *COMMON, "-c", path, "-o", obj]
    _run(cmd, verbose)
    return obj


# Measurement aid for bench.py (the device's practical read ceiling), a library of its own so
# that it is no part of libpagedkv's interface.
PROBE_SOURCES = ["read_ceiling.hip"]
PROBE_PATH = os.path.join(PKG_DIR, "libpkv_read_ceiling.so")


def _link(objs, path, verbose):
    tmp = path + ".tmp"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libpagedkv.so`` (and the benchmark's read-ceiling
    probe); returns the library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = HOST_SOURCES + DEVICE_SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(4, len(sources))) as ex:
        objs = dict(zip(sources, ex.map(lambda s: _compile(s, verbose), sources)))
    _link([objs[s] for s in HOST_SOURCES + DEVICE_SOURCES], LIB_PATH, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
