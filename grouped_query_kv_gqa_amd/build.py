"""Build libgqa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m grouped_query_kv_gqa_amd.build`` or ``build()``. Always
recompiles; objects go to ``grouped_query_kv_gqa_amd/_build/`` and the
library to ``grouped_query_kv_gqa_amd/libgqa.so``. The same sources built
with ``-DGQA_DEBUG`` (device range checks on every global access, see
``gqa_debug_checks``) give ``libgqa_debug.so``; the benchmark's bandwidth
probe goes to ``grouped_query_kv_gqa_amd/libgqa_probe.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa.so")
DEBUG_LIB = os.path.join(PKG, "libgqa_debug.so")  # range-checked build, for tests
PROBE_LIB = os.path.join(PKG, "libgqa_probe.so")  # bandwidth probe for the benchmark only

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++20", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only. Packed fp32 instructions are kept out of the
# generated code (the host pass warns that it does not know the feature).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]

SOURCES = ["decode.hip", "decode_noalloc.hip", "prefill.hip", "mean_pool.hip", "gqa_api.cpp", "plan.cpp",
           "workspace.cpp"]


def _compile(job) -> str:
    src, debug = job
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, ("debug_" if debug else "") + src + ".o")
    flags = [*COMMON, "-DGQA_DEBUG"] if debug else COMMON
    if src.endswith(".hip"):
        cmd = [HIPCC, *flags, *DEVICE, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *flags, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, debug) for debug in (False, True) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], DEBUG_LIB, verbose)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """The benchmark's HBM bandwidth probe, a separate small library."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMMON, *DEVICE, "-shared", os.path.join(CSRC, "hbm_probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for hbm_probe.hip:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
