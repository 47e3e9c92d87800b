"""Build libsmqa.so (gfx950) in-tree with hipcc.

    python -m fp8_kv_cache_sparse_amd.build

The decode path's translation units under csrc/ are compiled for gfx950 only and
linked into fp8_kv_cache_sparse_amd/libsmqa.so next to this file, and once more with
SMQA_DEBUG defined into libsmqa_debug.so (the same library with the device-side range
checks reported by smqa_debug_flags); the benchmark's streaming-read reference
(bench_read.hip) goes into libsmqa_bench.so beside them.
Packed-fp32 VALU instructions are disabled for the device code generation.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsmqa.so")
BENCH_LIB = os.path.join(PKG, "libsmqa_bench.so")
DEBUG_LIB = os.path.join(PKG, "libsmqa_debug.so")
SOURCES = ["api.hip", "score.hip", "topk.hip", "attend.hip", "attend_sd.hip"]
BENCH_SOURCES = ["bench_read.hip", "bench_fp8_mfma.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 target feature; drop that one warning
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, list(extra_flags), "") for s in SOURCES + BENCH_SOURCES]
    jobs += [(s, list(extra_flags) + ["-DSMQA_DEBUG=1"], "_debug") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), 16)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n, nb = len(SOURCES), len(BENCH_SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + nb], BENCH_LIB)
    _link(objs[n + nb:], DEBUG_LIB)
    if verbose:
        print(f"built {LIB}, {DEBUG_LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    extra = sys.argv[1:]
    build(extra, verbose=True)
