"""GPU parity of the block-scaled MFMA path of the MXFP4 bank (MXFP8 activations)
against the oracle, through the C-ABI.

Bars: the MXFP8 quantization (an integer decision: codes and scale bytes) bit-exact,
both sides taking it from the exact scaled value; the projections within the bf16
tolerance (max relative row error 2e-2) -- products are exact on both sides and
only the fp32 vs fp64 summation differs before the bf16 rounding.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, TOL, f64, row_rel_err
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, to_storage

pytestmark = pytest.mark.gpu


def test_mx8_quantize_bit_exact():
    print("[mx8_quantize]", flush=True)
    rng = np.random.default_rng(95)
    rows, K = 67, 2880
    mag = np.repeat(10.0 ** rng.uniform(-8, 8, size=(rows, K // 32)), 32, axis=1)
    x = rng.normal(0, 1, (rows, K)) * mag
    x[3, :32] = 0.0                                   # a zero block
    x[4, :32] = -1e-30                                # tiny negatives
    x[5, 32:64] = 448.0 * 1.07                        # values that saturate
    x[5, 32] = 479.0
    xb = to_storage(x, "bf16")
    q, s = moeq.mx8_quantize(di.tensor(xb, "bf16", DEV))
    torch.cuda.synchronize()
    rq, rs = oracle.mxfp8_quantize(xb, "bf16")
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def routed(T, seed=None, **over):
    cfg = dataclasses.replace(CONFIGS["mxfp4"], **over) if over else CONFIGS["mxfp4"]
    p = make_inputs(cfg, seed=seed, T=T)
    d = di.upload(p, DEV)
    disp = moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"])
    sel, _ = oracle.route(p["logits"], p["router_bias"], p["k"])
    _, src, _, rex = oracle.dispatch_index(sel, p["E"])
    return p, d, disp, src, rex


def gate_up_reference(p, values, rex, fn):
    q, s = oracle.mxfp8_quantize(values, "bf16")
    gu = oracle.mx8_project(q, s, rex, p["gu_blocks"], p["gu_scales"], p["gu_bias"], "bf16")
    return oracle.swiglu(gu[:, 0::2], gu[:, 1::2], "bf16", **fn)


def down_reference(p, h, rex):
    q, s = oracle.mxfp8_quantize(h, "bf16")
    return oracle.mx8_project(q, s, rex, p["dn_blocks"], p["dn_scales"], p["dn_bias"], "bf16")


FN = dict(clamp=7.0, alpha=1.0, up_offset=0.0)
ONE_SIDED = dict(clamp=7.0, alpha=1.702, up_offset=1.0, gate_one_sided=True)


@pytest.mark.parametrize("T,fn,over", [
    (24, FN, {}),
    (37, ONE_SIDED, {}),                       # ragged m-tiles, the one-sided variant
    (300, FN, dict(E=8, k=2)),                 # several full m-tiles per expert
])
def test_mx8_path_parity(T, fn, over):
    print(f"[mx8 path] T={T} fn={fn} {over}", flush=True)
    p, d, disp, src, rex = routed(T, **over)
    r = disp["route"]
    h = moeq.mx8_grouped_swiglu(r, disp["values"], d["gate"], **fn)
    values = oracle.copy_rows(p["x"], src)
    href = gate_up_reference(p, values, rex, {k: v for k, v in fn.items()})
    torch.cuda.synchronize()
    assert row_rel_err(f64(di.to_host(h, "bf16"), "bf16"), f64(href, "bf16")) <= TOL["bf16"]
    y = moeq.mx8_grouped_down(r, di.tensor(href, "bf16", DEV), d["down"])   # identical input
    torch.cuda.synchronize()
    yref = down_reference(p, href, rex)
    assert row_rel_err(f64(di.to_host(y, "bf16"), "bf16"), f64(yref, "bf16")) <= TOL["bf16"]


def test_mx8_full_size_sampled():
    """The whole MXFP4 workload (2048 tokens, top 4 of 128) in the launch shape the
    bench times; the oracle evaluates sampled rows (each row stands alone)."""
    print("[mx8 full size]", flush=True)
    p, d, disp, src, rex = routed(CONFIGS["mxfp4"].T)
    r = disp["route"]
    h = moeq.mx8_grouped_swiglu(r, disp["values"], d["gate"], **FN)
    y = moeq.mx8_grouped_down(r, h, d["down"])
    torch.cuda.synchronize()
    A = p["T"] * p["k"]
    rows = np.sort(np.random.default_rng(96).choice(A, 40, replace=False))
    values = oracle.copy_rows(p["x"], src)
    href = gate_up_reference(p, values[rows], rex[rows], FN)
    hg = di.to_host(h, "bf16")
    assert row_rel_err(f64(hg[rows], "bf16"), f64(href, "bf16")) <= TOL["bf16"]
    yref = down_reference(p, hg[rows], rex[rows])                            # the GPU's own h
    assert row_rel_err(f64(di.to_host(y, "bf16")[rows], "bf16"), f64(yref, "bf16")) <= TOL["bf16"]
