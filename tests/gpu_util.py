"""Helpers for the GPU parity tests (the oracle is the reference)."""
import numpy as np
import torch

from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import storage_to_f64

DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}   # max relative error: fp32 / bf16 activations


def row_rel_err(got, ref):
    """max over rows of ||got_t - ref_t||_inf / ||ref_t||_inf (float64)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.max(np.abs(got - ref), axis=1) / den)) if ref.size else 0.0


def f64(a, dt):
    return storage_to_f64(np.asarray(a), dt)


def run_path(p, d=None):
    """Run the whole HIP path on an inputs dict; return host copies of every output."""
    if d is None:
        d = di.upload(p, DEV)
    disp = moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"])
    r = disp["route"]
    h = moeq.awq_grouped_swiglu(r, disp["values"], d["gate"], d["up_arg"], p["clamp"],
                                p["alpha"], p["up_offset"],
                                gate_one_sided=p.get("gate_one_sided", False))
    y = moeq.awq_grouped_down(r, h, d["down"])
    out = moeq.moe_combine(r, y, disp["weights"])
    torch.cuda.synchronize()
    adt = p["adt"]
    return dict(selected=disp["selected"].cpu().numpy().view(np.uint32),
                weights=disp["weights"].cpu().numpy(),
                row_experts=disp["row_experts"].cpu().numpy().view(np.uint32),
                values=di.to_host(disp["values"], adt), h=di.to_host(h, adt),
                y=di.to_host(y, adt), out=di.to_host(out, adt),
                offsets=r.expert_offsets.cpu().numpy(), row_src=r.row_src.cpu().numpy(),
                slot_pos=r.slot_pos.cpu().numpy(), route=r, dev=d, disp=disp,
                h_dev=h, y_dev=y)
