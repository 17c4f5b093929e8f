"""The oracle and the library's host-side validation code under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

Each leg rebuilds one sanitized library and runs existing CPU tests against it in a
child process with the matching runtime preloaded (gcc's libasan for the oracle,
which gcc builds; clang's for the library's host code, which hipcc builds).  A
sanitizer report aborts the child (recovery is off), so the leg fails on any
out-of-bounds access, use after free, signed overflow, misaligned or null access or
invalid shift in the code under test.  Leak checking is off: the Python
interpreter itself holds allocations until exit.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

ORACLE_TESTS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
HOST_TESTS = [os.path.join(ROOT, "tests", "test_abi_host.py")]
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    for rep in REPORTS:
        assert rep not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out, out[-2000:]
    return out


def _gcc_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return hits[-1]


def _instrumented(lib):
    syms = subprocess.run(["nm", "-u", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms, lib
    assert "__ubsan_handle_" in syms, lib


def test_oracle_under_sanitizers():
    runtime = _gcc_runtime()
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    try:
        _instrumented(lib)
        out = _run(ORACLE_TESTS, {"LD_PRELOAD": runtime, "MOEQ_ORACLE_SANITIZE": "1"})
        assert "failed" not in out
    finally:
        os.remove(lib)


def test_host_validation_under_sanitizers():
    """The library built this way is as large as the product library and only
    serves this test, so it is removed afterwards."""
    runtime = _clang_runtime()
    from quantized_moe_expert_router_amd import build as pb
    lib = pb.build_host_sanitized()
    try:
        _instrumented(lib)
        out = _run(HOST_TESTS, {"LD_PRELOAD": runtime, "MOEQ_LIB": lib})
        assert "failed" not in out
    finally:
        os.remove(lib)
