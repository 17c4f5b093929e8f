"""fp16 activations and gradients through the C-ABI, against the oracle.

The pages let the activation storage differ from the scales' (frozen_awq:
FrozenAwqOps, the input storage).  fp16 rows run on the fp32 VALU kernels with
the same rounding points as the oracle: coefficients rounded to the scale dtype,
G, U, h, y and out rounded to fp16.

Tolerance: the kernels accumulate in fp32, the oracle in double, and both round
once to fp16 at each storage point, so a stored value may differ by one fp16 ulp
(2^-11 relative) where the two sums fall on either side of a rounding boundary;
through G, U -> h -> y that stays within a few ulps of a row's largest value.
5e-3 (about ten ulps) is the bound, well below what a dropped term or a
transposed operand gives.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, f64, row_rel_err, run_path
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, to_storage

pytestmark = pytest.mark.gpu

TOL16 = 5e-3

CASES = {
    "tiny-f16-scales": dataclasses.replace(CONFIGS["tiny"], adt="f16"),
    "tiny-bf16-scales": dataclasses.replace(CONFIGS["tiny"], adt="f16", sdt="bf16"),
    "tiny-f32-scales-bias": dataclasses.replace(CONFIGS["tiny"], adt="f16", sdt="f32",
                                                awq_bias=True),
    "decode-clamped": dataclasses.replace(CONFIGS["decode"], T=12, adt="f16", clamp=2.0),
    "mxfp4-bank": dataclasses.replace(CONFIGS["mxfp4"], T=6, adt="f16"),
}


def check_routing(p, g):
    sel, w = oracle.route(p["logits"], p["router_bias"], p["k"])
    off, src, pos, rex = oracle.dispatch_index(sel, p["E"])
    np.testing.assert_array_equal(g["selected"], sel)
    np.testing.assert_array_equal(g["slot_pos"], pos)
    np.testing.assert_array_equal(g["row_experts"], rex)
    np.testing.assert_array_equal(g["values"], oracle.copy_rows(p["x"], src))
    return pos, rex


@pytest.mark.parametrize("case", list(CASES))
def test_forward_fp16(case):
    cfg = CASES[case]
    p = make_inputs(cfg)
    print(f"[fp16 forward] {case} T={p['T']} H={p['H']} I={p['I']} E={p['E']}", flush=True)
    g = run_path(p)
    pos, _ = check_routing(p, g)
    ref = oracle.moe_forward(p)
    assert row_rel_err(f64(g["h"], "f16"), f64(ref["h"], "f16")) <= TOL16
    h_or = di.tensor(ref["h"], "f16", DEV)
    y_gpu = di.to_host(moeq.awq_grouped_down(g["route"], h_or, g["dev"]["down"]), "f16")
    assert row_rel_err(f64(y_gpu, "f16"), f64(ref["y"], "f16")) <= TOL16
    assert row_rel_err(f64(g["out"], "f16"), f64(ref["out"], "f16")) <= TOL16
    # the combine is bit-exact on identical y and weights
    out_c = moeq.moe_combine(g["route"], di.tensor(ref["y"], "f16", DEV), g["disp"]["weights"])
    np.testing.assert_array_equal(di.to_host(out_c, "f16"),
                                  oracle.combine(ref["y"], "f16", g["weights"], pos))


@pytest.mark.parametrize("case", ["tiny-f16-scales", "tiny-f32-scales-bias", "decode-clamped"])
def test_backward_fp16(case):
    """COPY VJP and combine VJP bit-exact; the chain input VJP within the fp16 bound."""
    cfg = CASES[case]
    p = make_inputs(cfg)
    print(f"[fp16 backward] {case}", flush=True)
    g = run_path(p)
    pos, rex = check_routing(p, g)
    A, H, T = p["T"] * p["k"], p["H"], p["T"]
    d, r = g["dev"], g["route"]
    rng = np.random.default_rng(71)
    gout = to_storage(rng.normal(0, 1, (T, H)), "f16")
    gy, gw = moeq.moe_combine_backward(r, g["y_dev"], g["disp"]["weights"],
                                       di.tensor(gout, "f16", DEV))
    grad = to_storage(rng.normal(0, 1, (A, H)), "f16")
    fn = (p["clamp"], p["alpha"], p["up_offset"])
    gv = moeq.awq_swiglu_input_backward(r, g["disp"]["values"], d["gate"], d["up"], d["down"],
                                        di.tensor(grad, "f16", DEV), *fn)
    gx = moeq.moe_dispatch_backward(r, di.tensor(grad, "f16", DEV))
    torch.cuda.synchronize()
    ry, _ = oracle.combine_backward(g["y"], "f16", g["weights"], pos, gout)
    np.testing.assert_array_equal(di.to_host(gy, "f16"), ry)
    np.testing.assert_array_equal(di.to_host(gx, "f16"), oracle.dispatch_backward(grad, "f16", pos))
    sdt, grp = p["sdt"], p["group"]
    dh = oracle.awq_input_backward(grad, "f16", rex, p["down_qw"], p["down_qz"], p["down_s"],
                                   sdt, grp)
    gate = (p["gate_qw"], p["gate_qz"], p["gate_s"], p["gate_b"])
    up = (p["up_qw"], p["up_qz"], p["up_s"], p["up_b"])
    rv = oracle.awq_swiglu_input_backward(g["values"], "f16", rex, gate, up, sdt, grp, dh, *fn)
    assert row_rel_err(f64(di.to_host(gv, "f16"), "f16"), f64(rv, "f16")) <= TOL16
    # the down input VJP alone
    dh_gpu = moeq.awq_input_backward(r, di.tensor(grad, "f16", DEV), d["down"])
    torch.cuda.synchronize()
    assert row_rel_err(f64(di.to_host(dh_gpu, "f16"), "f16"), f64(dh, "f16")) <= TOL16


def test_unsorted_rows_fp16():
    """Rows in any order (awq_expert_forward) with fp16 rows: each row with its own
    expert, against the oracle's projection of the same rows."""
    cfg = CASES["tiny-bf16-scales"]
    p = make_inputs(cfg)
    print("[fp16 unsorted]", flush=True)
    d = di.upload(p, DEV)
    rng = np.random.default_rng(72)
    rows = 40
    xh = to_storage(rng.normal(0, 1, (rows, p["H"])), "f16")
    ids = rng.integers(0, p["E"], rows).astype(np.uint32)
    y = moeq.awq_expert_forward(di.tensor(xh, "f16", DEV),
                                torch.from_numpy(ids.astype(np.int32)).to(DEV), d["gate"])
    torch.cuda.synchronize()
    ref = oracle.awq_project(xh, "f16", ids, p["gate_qw"], p["gate_qz"], p["gate_s"],
                             p["sdt"], p["group"], bias=p["gate_b"])
    assert row_rel_err(f64(di.to_host(y, "f16"), "f16"), f64(ref, "f16")) <= TOL16
