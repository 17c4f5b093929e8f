"""Build libmoeq.so (the HIP library behind include/moeq.h) for gfx950, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(CSRC, "libmoeq.so")
PEAKS_LIB = os.path.join(CSRC, "libmoeq_peaks.so")
PEAKS_SOURCE = "peaks.hip"
SOURCES = ["api.cpp", "route.hip", "gemm_generic.hip", "gemm_mfma.hip", "gemm_tile.hip", "gemm_wave.hip", "gemm_mx.hip", "gemm_ws.hip",
           "backward.hip", "gemm_vjp.hip",
           "gemm_mx8.hip", "static_route.hip"]
ARCH = os.environ.get("MOEQ_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         # packed fp32 arithmetic stays off (the device pass honours this feature;
         # the host pass warns that it does not know it)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, flush=True)
    return obj


def _link(objs, lib, verbose):
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", *objs, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + [PEAKS_SOURCE]))
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], PEAKS_LIB, verbose)   # measurement support for the benchmark
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
