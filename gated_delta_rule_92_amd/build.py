"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m gated_delta_rule_92_amd.build [--jobs N] [--verbose]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libkda.so")
# the HBM copy probe bench.py times beside the spec peak (measurement only,
# not part of the library)
PROBE_SRC = os.path.join(ROOT, "bench_hbm.hip")
PROBE_PATH = os.path.join(ROOT, "libhbm_probe.so")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_gate.hip", "kda_recurrent.hip", "kda_chunk.hip", "kda_chunk_pipe.hip", "kda_backward.hip",
           "kda_compose.hip", "kda_epilogue.hip"]

# Packed fp32 VALU instructions are disabled for every device compile.
# Matrix-core results are kept in ordinary VGPRs (-amdgpu-mfma-vgpr-form), which
# avoids accumulator-register copies.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build_probe(verbose: bool = False) -> str:
    """libhbm_probe.so: the hand-written HBM copy bench.py measures."""
    tmp = PROBE_PATH + ".tmp"
    cmd = [hipcc(), "-x", "hip", "-shared", PROBE_SRC, "-o", tmp] + COMMON_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        probe = ex.submit(build_probe, verbose)
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        probe.result()
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    sys.exit(main())
