"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python -m tiled_online_softmax_fa_amd.build  (or build() from Python).
Every call recompiles every source; objects go to _build/, the shared
libraries next to this file: libfa.so and the checking builds (same ABI,
built with one debug option each).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

SOURCES = ["fa_api.cpp", "fa_fwd_bf16.hip", "fa_fwd_f32.hip", "fa_bwd_bf16.hip", "fa_quant_fp8.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # NaN never occurs on the valid paths; this lets fmaxf lower to a bare
    # v_max/v_max3 without canonicalisation. Infinities stay honoured (-inf
    # is the mask value).
    "-fno-honor-nans",
    # no packed-fp32 VALU forms anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa")
    return path


# Checking builds, each a library of its own next to libfa.so with the same
# C ABI: their results must equal libfa.so's bit for bit (tests/
# test_gpu_checking_builds.py).
#   libfa_revgrid.so  workgroups take their tiles in reverse launch order
#   libfa_sync.so     every wait for the asynchronous K/V copies is a full wait
CHECK_BUILDS = {
    "revgrid": ["-DFA_REVERSE_GRID"],
    "sync": ["-DFA_DEBUG_SYNC"],
}


def check_lib_path(name: str) -> str:
    return os.path.join(PKG_DIR, f"libfa_{name}.so")


def _compile(src: str, verbose: bool, variant: str = "", defines=()) -> str:
    obj = os.path.join(BUILD_DIR, variant, os.path.splitext(src)[0] + ".o")
    os.makedirs(os.path.dirname(obj), exist_ok=True)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *HIPCC_FLAGS, *defines, "-I", INCLUDE, "-I", CSRC, *lang, "-c", os.path.join(CSRC, src), "-o",
           obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False, check_builds: bool = True) -> str:
    """Compile every source and link libfa.so (and the checking builds). Returns libfa.so's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    variants = [("", (), LIB_PATH)]
    if check_builds:
        variants += [(name, tuple(d), check_lib_path(name)) for name, d in CHECK_BUILDS.items()]
    jobs = [(src, v, d) for v, d, _ in variants for src in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs))
    for i, (_, _, path) in enumerate(variants):
        _link(objs[i * len(SOURCES):(i + 1) * len(SOURCES)], path, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
