"""moe_dispatch_static (the entry point for callers that cannot allocate) against
moe_dispatch with a caller workspace, through the C-ABI.

Bar: bit-exact (routing, dispatch order and row copies are integer and byte
work; the rest of the path then runs the same kernels on the same inputs).
Two calls in a row, the second with a smaller batch, so the second must not see
the first call's row mappings; plus the size limit and a failed call leaving the
route untouched.
"""
import ctypes as C
import dataclasses
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

_hip = None


def device_ints(ptr, n):
    """n int32 values at a device address (a host copy after a device sync)."""
    global _hip
    if _hip is None:
        _hip = C.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        _hip.hipMemcpy.restype = C.c_int
        _hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
    out = np.zeros(max(n, 1), np.int32)
    torch.cuda.synchronize()
    assert _hip.hipMemcpy(out.ctypes.data, C.c_void_p(ptr), 4 * n, 2) == 0  # device to host
    return out[:n]


def run(p, d, static):
    disp = (moeq.moe_dispatch_static if static else moeq.moe_dispatch)(
        d["x"], d["logits"], d["router_bias"], p["k"])
    r = disp["route"]
    h = moeq.awq_grouped_swiglu(r, disp["values"], d["gate"], d["up_arg"], p["clamp"])
    y = moeq.awq_grouped_down(r, h, d["down"])
    out = moeq.moe_combine(r, y, disp["weights"])
    torch.cuda.synchronize()
    A = p["T"] * p["k"]
    res = {k: disp[k].clone() for k in ("values", "weights", "selected", "row_experts")}
    res.update(out=out, h=h,
               offsets=device_ints(r.c.expert_offsets, p["E"] + 1),
               row_src=device_ints(r.c.row_src, A), slot_pos=device_ints(r.c.slot_pos, A),
               counts=moeq.moe_dispatch_counts(r, list(range(p["E"] + 1))))
    return res


@pytest.mark.parametrize("name,T1,T2", [("decode", 64, 40), ("prefill", 1024, 300),
                                        ("many", 1024, 256), ("mxfp4", 256, 33)])
def test_static_dispatch_matches_workspace_dispatch(name, T1, T2):
    for T in (T1, T2):
        print(f"[no-alloc dispatch] {name} T={T}", flush=True)
        p = make_inputs(dataclasses.replace(CONFIGS[name], T=T))
        d = di.upload(p, DEV)
        got = run(p, d, static=True)
        ref = run(p, d, static=False)
        for key in ("values", "weights", "selected", "row_experts", "h", "out"):
            assert torch.equal(got[key], ref[key]), (T, key)
        for key in ("offsets", "row_src", "slot_pos"):
            np.testing.assert_array_equal(got[key], ref[key])
        assert got["counts"] == ref["counts"] and sum(got["counts"]) == T * p["k"]


def test_static_dispatch_limit_and_failure_leave_route():
    x = torch.zeros(64, 256, dtype=torch.bfloat16, device=DEV)
    logits = torch.randn(64, 128, device=DEV)
    disp = moeq.moe_dispatch_static(x, logits, None, 8)
    before = bytes(disp["route"].c)
    # a batch whose route needs more than the static array holds
    T = 400000
    need = moeq.lib().moeq_route_workspace_bytes(T, 512, 10)
    assert need > (4 << 20)
    L, r = moeq.lib(), disp["route"]
    st = L.moe_dispatch_static(None, moeq.BF16, T, 256, None, moeq.F32, 512, None, 10, None,
                               None, None, None, C.byref(r.c), None)
    assert st == moeq.EWORKSPACE and b"static route array" in L.moeq_last_error()
    # invalid arguments: nothing enqueued, route untouched
    st = L.moe_dispatch_static(C.c_void_p(x.data_ptr()), 7, 64, 256,
                               C.c_void_p(logits.data_ptr()), moeq.F32, 128, None, 8, None, None,
                               None, None, C.byref(r.c), None)
    assert st == moeq.EDTYPE
    assert bytes(r.c) == before
    torch.cuda.synchronize()
