"""GPU checks of the autograd layer (quantized_moe_expert_router_amd.autograd).

* The forward output and torch.autograd.grad's derivatives are bit-identical to
  the C-ABI calls made directly in the same order (the layer only marshals).
* Against the oracle: the input derivative within the chain tolerance (max
  relative row error 1e-4 fp32 / 2e-2 bf16), the logit derivative bit-exact
  against the oracle's logit VJP of the GPU's weight derivative, which itself is
  within the combine-VJP bound of the oracle's (fp64 sums in another order,
  one rounding).
* create_graph=True raises HigherDerivativeUnsupported (packed_experts.rs
  PackedExpertAutodiffError); frozen_awq and packed_expert give the input VJP of
  frozen_awq.rs / packed_experts.rs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, TOL, f64, row_rel_err
from quantized_moe_expert_router_amd import autograd as ag
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, to_storage

pytestmark = pytest.mark.gpu

CASES = [("tiny", None, (0.0, 1.0, 0.0, False)),
         ("tiny", None, (1.5, 1.702, 1.0, True)),
         ("decode", None, (0.0, 1.0, 0.0, False)),
         ("prefill", 256, (0.0, 1.0, 0.0, False)),
         ("many", 128, (0.0, 1.0, 0.0, False)),
         ("decode", 64, (7.0, 1.0, 0.0, False))]


def direct(p, d, gout, fn):
    """The forward and backward calls made one by one."""
    clamp, alpha, off, one = fn
    disp = moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"])
    r = disp["route"]
    h = moeq.awq_grouped_swiglu(r, disp["values"], d["gate"], d["up_arg"], clamp, alpha, off,
                                gate_one_sided=one)
    y = moeq.awq_grouped_down(r, h, d["down"])
    out = moeq.moe_combine(r, y, disp["weights"])
    gy, gw = moeq.moe_combine_backward(r, y, disp["weights"], gout)
    gv = moeq.awq_swiglu_input_backward(r, disp["values"], d["gate"], d["up"], d["down"], gy,
                                        clamp, alpha, off, gate_one_sided=one)
    gx = moeq.moe_dispatch_backward(r, gv)
    gl = moeq.moe_dispatch_weights_backward(r, disp["selected"], disp["weights"], gw)
    return dict(out=out, y=y, gy=gy, gw=gw, gx=gx, gl=gl, disp=disp)


@pytest.mark.parametrize("name,T,fn", CASES)
def test_autograd_matches_calls_and_oracle(name, T, fn):
    print(f"[autograd] {name} T={T} fn={fn}", flush=True)
    cfg = CONFIGS[name] if T is None else dataclasses.replace(CONFIGS[name], T=T)
    p = make_inputs(cfg)
    adt = p["adt"]
    d = di.upload(p, DEV)
    gout_h = to_storage(np.random.default_rng(60).normal(0, 1, (p["T"], p["H"])), adt)
    gout = di.tensor(gout_h, adt, DEV)
    x = d["x"].clone().requires_grad_(True)
    logits = d["logits"].clone().requires_grad_(True)
    out = ag.moe_expert_ffn(x, logits, d["gate"], d["up_arg"], d["down"], p["k"],
                            expert_bias=d["router_bias"], clamp=fn[0], alpha=fn[1],
                            up_offset=fn[2], gate_one_sided=fn[3])
    gx, gl = torch.autograd.grad(out, (x, logits), gout)
    ref = direct(p, d, gout, fn)
    torch.cuda.synchronize()
    assert torch.equal(out, ref["out"])
    assert torch.equal(gx, ref["gx"]) and torch.equal(gl, ref["gl"])
    assert gx.dtype == x.dtype and gl.dtype == torch.float32

    # against the oracle, on the GPU's own expert rows y
    sel, w = oracle.route(p["logits"], p["router_bias"], p["k"])
    _, src, pos, rex = oracle.dispatch_index(sel, p["E"])
    y = di.to_host(ref["y"], adt)
    ry, rw = oracle.combine_backward(y, adt, w, pos, gout_h)
    np.testing.assert_array_equal(di.to_host(ref["gy"], adt), ry)
    gw = ref["gw"].cpu().numpy()
    yf, gf = np.abs(f64(y, adt)), np.abs(f64(gout_h, adt))
    absdot = np.stack([np.sum(gf * yf[pos[:, j]], axis=1) for j in range(p["k"])], axis=1)
    assert np.all(np.abs(gw.astype(np.float64) - rw) <= 2.0 ** -22 * np.abs(rw)
                  + 2.0 ** -38 * absdot)
    np.testing.assert_array_equal(gl.cpu().numpy(),
                                  oracle.dispatch_weights_backward(sel, w, gw, p["E"]))
    values = oracle.copy_rows(p["x"], src)
    sdt, g = p["sdt"], p["group"]
    dh = oracle.awq_input_backward(ry, adt, rex, p["down_qw"], p["down_qz"], p["down_s"], sdt, g)
    rv = oracle.awq_swiglu_input_backward(values, adt, rex,
                                          (p["gate_qw"], p["gate_qz"], p["gate_s"], p["gate_b"]),
                                          (p["up_qw"], p["up_qz"], p["up_s"], p["up_b"]),
                                          sdt, g, dh, fn[0], fn[1], fn[2], fn[3])
    rx = oracle.dispatch_backward(rv, adt, pos)
    assert row_rel_err(f64(di.to_host(gx, adt), adt), f64(rx, adt)) <= TOL[adt]


def test_autograd_logits_only_and_bank():
    """Only the logits need a derivative: the chain VJP is skipped; MXFP4 banks
    take this path (their input VJP is not implemented)."""
    print("[autograd] mxfp4 logits only", flush=True)
    cfg = dataclasses.replace(CONFIGS["mxfp4"], T=64)
    p = make_inputs(cfg)
    d = di.upload(p, DEV)
    logits = d["logits"].clone().requires_grad_(True)
    out = ag.moe_expert_ffn(d["x"], logits, d["gate"], None, d["down"], p["k"],
                            clamp=p["clamp"])
    gout_h = to_storage(np.random.default_rng(61).normal(0, 1, (p["T"], p["H"])), "bf16")
    (gl,) = torch.autograd.grad(out, (logits,), di.tensor(gout_h, "bf16", DEV))
    disp = moeq.moe_dispatch(d["x"], d["logits"], None, p["k"])
    r = disp["route"]
    h = moeq.awq_grouped_swiglu(r, disp["values"], d["gate"], None, p["clamp"])
    y = moeq.awq_grouped_down(r, h, d["down"])
    _, gw = moeq.moe_combine_backward(r, y, disp["weights"], di.tensor(gout_h, "bf16", DEV),
                                      experts=False)
    ref = moeq.moe_dispatch_weights_backward(r, disp["selected"], disp["weights"], gw)
    torch.cuda.synchronize()
    assert torch.equal(gl, ref)


def test_autograd_higher_order_raises():
    print("[autograd] create_graph", flush=True)
    p = make_inputs(CONFIGS["tiny"])
    d = di.upload(p, DEV)
    x = d["x"].clone().requires_grad_(True)
    out = ag.moe_expert_ffn(x, d["logits"], d["gate"], d["up"], d["down"], p["k"])
    with pytest.raises(ag.PackedExpertAutodiffError) as ei:
        torch.autograd.grad(out, x, torch.ones_like(out), create_graph=True)
    assert ei.value.kind == "HigherDerivativeUnsupported"
    torch.cuda.synchronize()


@pytest.mark.parametrize("adt", ["bf16", "f32"])
def test_frozen_awq_and_packed_expert_autograd(adt):
    print(f"[autograd] frozen_awq / packed_expert {adt}", flush=True)
    cfg = dataclasses.replace(CONFIGS["decode"], T=48, E=4, H=256, I=128, group=64, adt=adt,
                              awq_bias=True)
    p = make_inputs(cfg, seed=62)
    d = di.upload(p, DEV)
    rows = 96
    rng = np.random.default_rng(63)
    xh = to_storage(rng.normal(0, 1, (2, rows // 2, cfg.H)), adt)
    gh = to_storage(rng.normal(0, 1, (2, rows // 2, cfg.I)), adt)
    g = d["gate"]
    one = moeq.AwqExperts(g.qweight[:1].contiguous(), g.qzeros[:1].contiguous(),
                          g.scales[:1].contiguous(), g.group_size, g.bias[:1].contiguous())
    x = di.tensor(xh, adt, DEV).requires_grad_(True)
    y = ag.frozen_awq(x, one)
    (gx,) = torch.autograd.grad(y, x, di.tensor(gh, adt, DEV))
    assert y.shape == (2, rows // 2, cfg.I) and gx.shape == x.shape
    want_y = moeq.frozen_awq_forward(x.detach().reshape(rows, -1), one)
    want_gx = moeq.awq_input_backward(None, di.tensor(gh, adt, DEV).reshape(rows, -1), one)
    ids = torch.from_numpy(rng.integers(0, cfg.E, rows).astype(np.int32)).to(DEV)
    x2 = x.detach().clone().requires_grad_(True)
    y2 = ag.packed_expert(x2, ids.reshape(2, -1), g)
    (gx2,) = torch.autograd.grad(y2, x2, di.tensor(gh, adt, DEV))
    want_y2 = moeq.awq_expert_forward(x.detach().reshape(rows, -1), ids, g)
    want_gx2 = moeq.awq_expert_input_backward(di.tensor(gh, adt, DEV).reshape(rows, -1), ids, g)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(rows, -1), want_y) and torch.equal(gx.reshape(rows, -1), want_gx)
    assert torch.equal(y2.reshape(rows, -1), want_y2)
    assert torch.equal(gx2.reshape(rows, -1), want_gx2)
    # the input VJP against the oracle (transpose of the same rounded coefficients)
    ref = oracle.awq_input_backward(gh.reshape(rows, -1), adt, ids.cpu().numpy().astype(np.uint32),
                                    p["gate_qw"], p["gate_qz"], p["gate_s"], p["sdt"], p["group"])
    assert row_rel_err(f64(di.to_host(gx2.reshape(rows, -1), adt), adt), f64(ref, adt)) <= TOL[adt]
