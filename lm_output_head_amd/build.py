"""Build libflashhead.so (and bench.py's libflashhead_bench.so) in-tree with
hipcc for gfx950.

Usage: ``python -m lm_output_head_amd.build``.
Every call compiles from source; object files go to ``lm_output_head_amd/_build``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashhead.so")
# bench.py --burst only: the plain read probe, outside the product's C ABI
BENCH_LIB = os.path.join(PKG, "libflashhead_bench.so")
BENCH_SOURCE = os.path.join(PKG, "bench_read_probe.hip")

SOURCES = ["fh_kernels.hip", "fh_mfma.hip", "fh_cluster.hip", "fh_batch1_bf16.hip", "fh_batch1_bf16_int4.hip",
           "fh_batch1_bf16_int8.hip", "fh_batch1_f32.hip", "fh_batch1_f32_int8.hip",
           "fh_batch1_f32_int4.hip", "fh_spec.hip", "fh_probs.hip", "fh_engine.cpp"]

# Packed FP32 instructions are disabled for all device code.
COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; ROCm is required to build libflashhead")
    return h


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link libflashhead.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, LIB)
    tmp = BENCH_LIB + ".tmp"
    cmd = [_hipcc(), *COMMON, *extra, "-shared", "-x", "hip", BENCH_SOURCE, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"bench library build failed: {' '.join(cmd)}\n{r.stdout}")
    os.replace(tmp, BENCH_LIB)
    if verbose:
        print(f"built {LIB} and {BENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
