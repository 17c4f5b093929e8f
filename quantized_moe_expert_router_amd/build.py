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
HOSTSAN_LIB = os.path.join(CSRC, "libmoeq_hostsan.so")
# the host-only validation code: api.cpp (every entry point's argument checks) and
# the static-route set-up; the kernels' files join the sanitized library unchanged
HOSTSAN_SOURCES = ["api.cpp", "static_route.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         # packed fp32 arithmetic stays off (the device pass honours this feature;
         # the host pass warns that it does not know it)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


def _compile(src: str, verbose: bool, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = ["hipcc", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
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


def build_host_sanitized(verbose: bool = False) -> str:
    """libmoeq_hostsan.so: the same library with its host-side validation code
    built under AddressSanitizer and UndefinedBehaviorSanitizer (clang's
    runtimes, host pass only; the device code is untouched).  For CPU tests of
    the argument checks: a process that loads it needs clang's
    libclang_rt.asan-x86_64.so first in LD_PRELOAD, and names it in MOEQ_LIB.
    Links the kernels' objects of the last build()."""
    san = ["-O1", "-g"]
    for f in ("address", "undefined"):
        san += ["-Xarch_host", f"-fsanitize={f}"]
    san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    rest = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o")
            for s in SOURCES if s not in HOSTSAN_SOURCES]
    missing = [o for o in rest if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing[0]} is missing")
    objs = [_compile(s, verbose, san, "_hostsan") for s in HOSTSAN_SOURCES]
    _link(objs + rest, HOSTSAN_LIB, verbose)
    return HOSTSAN_LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    if "--host-sanitized" in sys.argv:
        build_host_sanitized(verbose="-q" not in sys.argv)
