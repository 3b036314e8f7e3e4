"""Build the gfx950 HIP library ``libefla.so`` in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
one shared library next to this file. Always rebuilds when called.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libefla.so")

SOURCES = ["efla_api.hip", "efla_chunked.hip", "efla_decode.hip", "efla_backward.hip", "efla_noalloc.hip"]
# measurement-only kernels (achievable MFMA rate and streaming bandwidth),
# linked into a separate library that only the benchmark loads
BENCH_SOURCES = ["bench_peaks.hip"]
BENCH_LIB = os.path.join(PKG, "libefla_bench.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU ops on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no sinking of look-alike code out of the per-wave role branches into a
    # common successor: with it, the chunked kernel's tile-job dispatch was
    # compiled so that one wave stored its Q K^T tile through an address
    # register that was never set on its path (tile (1,0) of a 32-row chunk
    # landed on (1,1)); with each branch keeping its own stores, every store
    # has its constant offset
    "-mllvm", "-simplifycfg-sink-common=false",
    "-I", INCLUDE,
    "-I", CSRC,
]


# Per-file flags. The chunked forward's waves each run one dependent chain at
# fixed occupancy (one workgroup per CU), and the ILP-first machine scheduler
# orders those chains better than the default occupancy-first one (measured
# on one MI355X: 1.3B-layer shape 164.5 -> 160.0 us, 340M layer 88.2 -> 85.6
# us, no spills); on the backward's kernels it was slower, so they keep the
# default.
FILE_FLAGS = {"efla_chunked.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + BENCH_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in BENCH_SOURCES], BENCH_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
