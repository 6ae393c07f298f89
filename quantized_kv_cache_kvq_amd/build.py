"""Build libkvq.so in-tree with hipcc for gfx950.

    python -m quantized_kv_cache_kvq_amd.build      # or call build()

Each translation unit under csrc/ compiles to an object in _build/ (in
parallel), then the objects are linked into quantized_kv_cache_kvq_amd/libkvq.so.
The measurement kernels under probe/ (HBM stream read, matrix-core loop) are
linked apart into quantized_kv_cache_kvq_amd/libkvq_probe.so.  Packed FP32
vector instructions are disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "libkvq")
LIB = os.path.join(PKG, "libkvq.so")
PROBE_LIB = os.path.join(PKG, "libkvq_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Attention kernels: NaN inputs are outside the contract, so fmax needs no
# NaN canonicalization and max reductions fuse with their DPP moves.  Device
# code only: the host-side argument checks keep IEEE NaN semantics.
PER_FILE = {
    "kvq_decode.hip": ["-Xarch_device", "-fno-honor-nans"],
    "kvq_block.hip": ["-Xarch_device", "-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [hipcc(), *COMMON, *extra, "-I", INCLUDE, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {lib}:\n{r.stderr[-6000:]}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(PROBE, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(_compile, srcs + probes))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
