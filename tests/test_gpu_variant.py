"""GPU parity of the one-sided-clamp SwiGLU variant (gate clamped from above only,
sigmoid(1.702 g), u + 1 -- the form some MXFP4 models use) against the oracle,
through the C-ABI, forward and backward.  Bars as elsewhere: max relative row
error 1e-4 (fp32 activations) / 2e-2 (bf16).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, TOL, f64, row_rel_err, run_path
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, to_storage

pytestmark = pytest.mark.gpu

VARIANT = dict(clamp=7.0, alpha=1.702, up_offset=1.0, gate_one_sided=True)


def variant_inputs(name, T, **over):
    cfg = dataclasses.replace(CONFIGS[name], **over) if over else CONFIGS[name]
    p = make_inputs(cfg, T=T)
    p.update(VARIANT)
    return p


@pytest.mark.parametrize("name,T,over", [
    ("mxfp4", 24, {}),                        # MXFP4 bank kernel
    ("tiny", 16, {}),                         # fp32 activations
    ("decode", 64, {}),                       # stream kernel
    ("prefill", 96, {}),                      # stream kernel too: 6 rows per expert
    ("many", 80, {}),                         # fp32 scales, biases; stream kernel
])
def test_variant_forward(name, T, over):
    p = variant_inputs(name, T, **over)
    print(f"[variant forward] {name} T={T}", flush=True)
    g = run_path(p)
    ref = oracle.moe_forward(p)
    tol = TOL[p["adt"]]
    assert row_rel_err(f64(g["h"], p["adt"]), f64(ref["h"], p["adt"])) <= tol
    assert row_rel_err(f64(g["out"], p["adt"]), f64(ref["out"], p["adt"])) <= tol
    if name in ("decode", "prefill", "many"):
        # gate values below -7 occur at these shapes, so the variant differs from the
        # two-sided clamp on these inputs
        gu = [oracle.awq_project(ref["values"], p["adt"], ref["row_experts"], p[c + "_qw"],
                                 p[c + "_qz"], p[c + "_s"], p["sdt"], p["group"],
                                 bias=p[c + "_b"]) for c in ("gate", "up")]
        two = oracle.swiglu(gu[0], gu[1], p["adt"], clamp=7.0, alpha=1.702, up_offset=1.0)
        assert not np.array_equal(two, ref["h"])


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_variant_backward_chain(name):
    T = {"tiny": 16, "decode": 64, "prefill": 96}[name]
    p = variant_inputs(name, T)
    print(f"[variant backward] {name} T={T}", flush=True)
    d = di.upload(p, DEV)
    disp = moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"])
    sel, _ = oracle.route(p["logits"], p["router_bias"], p["k"])
    _, src, _, rex = oracle.dispatch_index(sel, p["E"])
    adt, A = p["adt"], p["T"] * p["k"]
    grad = to_storage(np.random.default_rng(81).normal(0, 1, (A, p["H"])), adt)
    gv = moeq.awq_swiglu_input_backward(disp["route"], disp["values"], d["gate"], d["up"],
                                        d["down"], di.tensor(grad, adt, DEV), 7.0, 1.702, 1.0,
                                        gate_one_sided=True)
    torch.cuda.synchronize()
    values = oracle.copy_rows(p["x"], src)
    dh = oracle.awq_input_backward(grad, adt, rex, p["down_qw"], p["down_qz"], p["down_s"],
                                   p["sdt"], p["group"])
    ref = oracle.awq_swiglu_input_backward(
        values, adt, rex, (p["gate_qw"], p["gate_qz"], p["gate_s"], p["gate_b"]),
        (p["up_qw"], p["up_qz"], p["up_s"], p["up_b"]), p["sdt"], p["group"], dh, 7.0, 1.702,
        1.0, gate_one_sided=True)
    assert row_rel_err(f64(di.to_host(gv, adt), adt), f64(ref, adt)) <= TOL[adt]


# The clamp epilogues of the MFMA kernels that serve many rows per expert.  At
# 128 rows per expert the stream kernel is out of the way (it takes at most 8),
# and each of the register-decoded (wave), warp-specialised (ws) and LDS-tiled
# (tile) kernels is forced on in turn by switching the ones before it off.  The
# clamp is set to 1.0 so that it binds on a good share of G and U at these sizes.
FNS = {"two-sided": (1.0, 1.0, 0.0, False), "one-sided": (1.0, 1.702, 1.0, True)}
KERNEL_CASES = {
    "wave": dict(T=512, E=8, k=2, H=512, I=256, sdt="bf16", awq_bias=False),
    "ws": dict(T=600, E=12, k=2, H=512, I=256, sdt="f32", awq_bias=True),
    "tile": dict(T=512, E=8, k=2, H=384, I=256, sdt="f16", awq_bias=True),
}


def force_kernel(kernel, monkeypatch):
    if kernel in ("ws", "tile"):
        monkeypatch.setenv("MOEQ_WAVE", "0")
    if kernel == "tile":
        monkeypatch.setenv("MOEQ_WS", "0")


def kernel_inputs(kernel, fn, **over):
    cfg = dataclasses.replace(CONFIGS["decode"], **{**KERNEL_CASES[kernel], **over})
    p = make_inputs(cfg, seed=90 + len(kernel))
    p.update(clamp=fn[0], alpha=fn[1], up_offset=fn[2], gate_one_sided=fn[3])
    return p


def clamp_share(p, ref):
    """Fraction of G and U entries beyond the clamp (oracle values)."""
    gu = [f64(oracle.awq_project(ref["values"], p["adt"], ref["row_experts"], p[c + "_qw"],
                                 p[c + "_qz"], p[c + "_s"], p["sdt"], p["group"],
                                 bias=p[c + "_b"]), p["adt"]) for c in ("gate", "up")]
    return [float(np.mean(np.abs(v) > p["clamp"])) for v in gu]


@pytest.mark.parametrize("fn", list(FNS))
@pytest.mark.parametrize("kernel", list(KERNEL_CASES))
def test_clamp_epilogue_forward(kernel, fn, monkeypatch):
    force_kernel(kernel, monkeypatch)
    p = kernel_inputs(kernel, FNS[fn])
    rows = p["T"] * p["k"] / p["E"]
    print(f"[clamp epilogue forward] {kernel} {fn} rows/expert={rows:.0f}", flush=True)
    assert rows >= 16
    g = run_path(p)
    ref = oracle.moe_forward(p)
    share = clamp_share(p, ref)
    assert all(0.05 < v < 0.95 for v in share), share
    tol = TOL[p["adt"]]
    assert row_rel_err(f64(g["h"], "bf16"), f64(ref["h"], "bf16")) <= tol
    assert row_rel_err(f64(g["out"], "bf16"), f64(ref["out"], "bf16")) <= tol


@pytest.mark.parametrize("fn", list(FNS))
@pytest.mark.parametrize("kernel", list(KERNEL_CASES))
def test_clamp_epilogue_backward(kernel, fn, monkeypatch):
    """The chain input VJP: the wave and ws kernels recompute G and U with the
    backward epilogue (clamp masks); with both off the chain runs two plain
    projections and the elementwise SwiGLU VJP.

    bf16 scales here, for every kernel: the clamp's derivative is a step, so G or
    U one rounding away on the other side of the bound changes a whole row of the
    result.  With bf16 scales the kernels' MFMA operands are the oracle's
    coefficients themselves; with fp32 or fp16 scales they are those
    coefficients rounded once more to bf16, which moves a few hundred of the
    ~600k G, U values across the bound at these sizes (a CPU emulation of that
    rounding gives the same 0.23 row error the kernels show)."""
    force_kernel(kernel, monkeypatch)
    c, alpha, off, one = FNS[fn]
    p = kernel_inputs(kernel, FNS[fn], sdt="bf16")
    print(f"[clamp epilogue backward] {kernel} {fn}", flush=True)
    d = di.upload(p, DEV)
    disp = moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"])
    sel, _ = oracle.route(p["logits"], p["router_bias"], p["k"])
    _, src, _, rex = oracle.dispatch_index(sel, p["E"])
    adt, A = p["adt"], p["T"] * p["k"]
    grad = to_storage(np.random.default_rng(91).normal(0, 1, (A, p["H"])), adt)
    gv = moeq.awq_swiglu_input_backward(disp["route"], disp["values"], d["gate"], d["up"],
                                        d["down"], di.tensor(grad, adt, DEV), c, alpha, off,
                                        gate_one_sided=one)
    torch.cuda.synchronize()
    values = oracle.copy_rows(p["x"], src)
    dh = oracle.awq_input_backward(grad, adt, rex, p["down_qw"], p["down_qz"], p["down_s"],
                                   p["sdt"], p["group"])
    ref = oracle.awq_swiglu_input_backward(
        values, adt, rex, (p["gate_qw"], p["gate_qz"], p["gate_s"], p["gate_b"]),
        (p["up_qw"], p["up_qz"], p["up_s"], p["up_b"]), p["sdt"], p["group"], dh, c, alpha,
        off, gate_one_sided=one)
    assert row_rel_err(f64(di.to_host(gv, adt), adt), f64(ref, adt)) <= TOL[adt]
