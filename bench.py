"""Benchmark: MoE expert-FFN tokens/s on one MI355X, with the roofline of the
dominant kernel and the CPU oracle timed beside it.

One step = the whole forward path over one batch: moe_dispatch (router top-k +
softmax + stable COPY dispatch) -> awq_grouped_swiglu -> awq_grouped_down ->
moe_combine.  Inputs are seeded synthetic tensors resident in HBM before the
timed region.  Each step reads a different replica of the expert weights (as
consecutive MoE layers would), so no step finds the previous step's weights in
the 256 MB last-level cache.  Steps are captured once as HIP graphs -- a whole
cycle over the replicas in one graph -- and replayed.

Prints ONE JSON line.  Default workload: the decode-shaped AWQ MoE
(T=64, hidden 2048, intermediate 768, 128 experts, top_k 8, group 128, bf16).

--path unsorted times awq_expert_forward (rows in any order with their global
expert IDs: local sort, grouped projection, inverse permutation) on the gate cube,
one row per assignment in token order -- the expert-parallel receive primitive.
The call validates the IDs on the host, so it synchronises and runs eagerly.

--path mx8 (MXFP4 workload only) times the same forward step with the bank on
gfx950's block-scaled MFMA: mx8_grouped_swiglu / mx8_grouped_down quantize their
input rows to MXFP8 and multiply them with the FP4 bank as stored -- an opt-in
variant whose activations are rounded differently from the bf16 path.

--path backward times the first-order backward path instead: one step =
moe_combine_backward (expert rows + FP32 weights) -> awq_swiglu_input_backward
(down VJP, recomputed gate/up with the SwiGLU VJP, both transposed cubes) ->
moe_dispatch_backward -> moe_dispatch_weights_backward, on the same workload,
with the forward's values, y and routing resident before the timed region.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "MoE expert-FFN tokens/s at 1 GPU; % of HBM (decode) / MFMA (prefill) peak"
METRIC_BWD = "MoE expert-FFN backward tokens/s at 1 GPU (first-order input VJPs)"
METRIC_MX8 = "MoE expert-FFN tokens/s at 1 GPU, MXFP4 bank on the block-scaled MFMA (MXFP8 activations)"
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA (the fp8 x fp4 scaled MFMA's operand type)
METRIC_UNSORTED = "unsorted-row expert projection rows/s at 1 GPU (gate cube, rows in token order)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="decode",
                    choices=["tiny", "decode", "prefill", "many", "mxfp4"])
    ap.add_argument("--replica-bytes", type=float, default=1.2e9,
                    help="weight bytes cycled through by consecutive steps")
    ap.add_argument("--path", default="forward",
                    choices=["forward", "backward", "unsorted", "mx8"])
    ap.add_argument("--eager", action="store_true", help="no HIP graph capture")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 launches): the "
                         "known-size reference that scales the HBM byte counters")
    return ap.parse_args()


def workload_name(cfg):
    kind = {"tiny": "tiny AWQ MoE FFN", "decode": "decode-shaped AWQ MoE FFN",
            "prefill": "prefill-shaped AWQ MoE FFN", "many": "many-expert AWQ MoE FFN",
            "mxfp4": "MXFP4 interleaved-bank MoE FFN"}[cfg.name]
    return (f"{kind}: T={cfg.T} hidden={cfg.H} intermediate={cfg.I} E={cfg.E} "
            f"top_k={cfg.k} group={cfg.group} act={cfg.adt} scales={cfg.sdt}")


def alg_bytes(p, offsets):
    """Algorithmic bytes of one step, from the actual routing.

    Weights: packed words, zeros, scales and bias of touched experts only.
    Activations: logits, x, values write+read, h write+read, y write+read,
    weights, out."""
    import numpy as np
    E, T, k, H, I = p["E"], p["T"], p["k"], p["H"], p["I"]
    A = T * k
    counts = np.diff(offsets)
    touched = int(np.count_nonzero(counts))
    ab = 4 if p["adt"] == "f32" else 2
    if p["fmt"] == "awq":
        sb = {"f32": 4, "f16": 2, "bf16": 2}[p["sdt"]]
        g = p["group"]

        def cube(K, N, bias):
            return K * N // 2 + (K // g) * (N // 8) * 4 + (K // g) * N * sb + (N * sb if bias else 0)
        gu_e = 2 * cube(H, I, p["gate_b"] is not None)
        dn_e = cube(I, H, p["down_b"] is not None)
    else:
        gu_e = 2 * I * (H // 32) * 17 + 2 * I * 2
        dn_e = H * (I // 32) * 17 + H * 2
    w_gu, w_dn = touched * gu_e, touched * dn_e
    act_gu = A * H * ab + A * I * ab                 # values read, h written
    act_dn = A * I * ab + A * H * ab                 # h read, y written
    act_other = T * E * 4 + T * H * ab + A * H * ab + T * k * 4 + A * H * ab + T * H * ab
    return dict(touched=touched, gateup=w_gu + act_gu, down=w_dn + act_dn,
                total=w_gu + w_dn + act_gu + act_dn + act_other, weights=w_gu + w_dn,
                w_gateup=w_gu, w_down=w_dn)


def flops(p):
    A = p["T"] * p["k"]
    return 6 * A * p["H"] * p["I"]


TRAFFIC_SOURCES = ("quantized_moe_expert_router_amd/csrc/gemm_mfma.hip",
                   "quantized_moe_expert_router_amd/csrc/awq_dequant.hpp",
                   "quantized_moe_expert_router_amd/csrc/common.hpp",
                   "quantized_moe_expert_router_amd/csrc/internal.hpp")


def kernel_digest():
    """Digest of the sources the gate/up stream kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config_name):
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counters), or
    None when there is none for this workload or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"awq_stream_kernel.{config_name}.traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_digest") != kernel_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(mib):
    """A plain device-to-device copy of known size, launched 5 times."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(cfg, target_s):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from quantized_moe_expert_router_amd.synth import make_inputs
    T = cfg.T if cfg.name in ("tiny", "decode") else min(cfg.T, 16)
    p = make_inputs(cfg, T=T)
    oracle._load()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_forward(p, keep_intermediates=False)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return {"value": round(reps * T / el, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x full forward of a {T}-token batch of this workload "
                      f"({el:.1f} s, double accumulation, OpenMP)"}


def cpu_baseline_backward(cfg, target_s):
    """The oracle's backward steps as they stand, on a bounded sample."""
    import numpy as np
    import oracle
    from quantized_moe_expert_router_amd.synth import make_inputs, to_storage
    T = cfg.T if cfg.name == "tiny" else min(cfg.T, 16)
    p = make_inputs(cfg, T=T)
    oracle._load()
    ref = oracle.moe_forward(p)
    adt, sdt, g = p["adt"], p["sdt"], p["group"]
    gout = to_storage(np.random.default_rng(5).normal(0, 1, (T, p["H"])), adt)
    gate = (p["gate_qw"], p["gate_qz"], p["gate_s"], p["gate_b"])
    up = (p["up_qw"], p["up_qz"], p["up_s"], p["up_b"])
    rex, pos = ref["row_experts"], ref["slot_pos"]
    reps, t0 = 0, time.perf_counter()
    while True:
        dy, dw = oracle.combine_backward(ref["y"], adt, ref["weights"], pos, gout)
        dh = oracle.awq_input_backward(dy, adt, rex, p["down_qw"], p["down_qz"], p["down_s"],
                                       sdt, g)
        dv = oracle.awq_swiglu_input_backward(ref["values"], adt, rex, gate, up, sdt, g, dh)
        oracle.dispatch_backward(dv, adt, pos)
        oracle.dispatch_weights_backward(ref["selected"], ref["weights"], dw, p["E"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return {"value": round(reps * T / el, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x full backward of a {T}-token batch of this workload "
                      f"({el:.1f} s, double accumulation, OpenMP)"}


def bwd_alg_bytes(p, ab_fwd):
    """Algorithmic bytes of the chain call: the touched down cube once and the
    touched gate/up cubes twice (the recompute of G, U reduces over the hidden
    features, the transposed product over the intermediate ones: two passes),
    plus values, grad and grad_values, and dh, dG, dU each written and read once."""
    A, H, I = p["T"] * p["k"], p["H"], p["I"]
    ab = 4 if p["adt"] == "f32" else 2
    return ab_fwd["w_down"] + 2 * ab_fwd["w_gateup"] + 3 * A * H * ab + 6 * A * I * ab


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path "
              "would shard by tokens or by expert ranges across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return

    import numpy as np
    import torch

    from quantized_moe_expert_router_amd import device_inputs as di
    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, weight_bytes

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moeq.lib()
    p = make_inputs(cfg)
    base = di.upload(p, dev)
    wb = weight_bytes(p)
    R = max(2, math.ceil(args.replica_bytes / wb))
    wkeys = ("gate", "up_arg", "down")

    def clone(w):
        if w is None:
            return None
        if isinstance(w, moeq.AwqExperts):
            return moeq.AwqExperts(w.qweight.clone(), w.qzeros.clone(), w.scales.clone(),
                                   w.group_size, None if w.bias is None else w.bias.clone())
        return moeq.Mxfp4Bank(w.blocks.clone(), w.scales.clone(), w.bias.clone(),
                              w.interleaved_gate_up)
    replicas = [{k: base[k] for k in wkeys}] + [{k: clone(base[k]) for k in wkeys}
                                               for _ in range(R - 1)]

    T, k, H, I, E = cfg.T, cfg.k, cfg.H, cfg.I, cfg.E
    A = T * k
    adt = base["x"].dtype
    route = moeq.RouteState(T, E, k, dev)
    bufs = dict(values=torch.empty(A, H, dtype=adt, device=dev),
                weights=torch.empty(T, k, dtype=torch.float32, device=dev),
                selected=torch.empty(T, k, dtype=torch.int32, device=dev),
                row_experts=torch.empty(A, dtype=torch.int32, device=dev))
    h = torch.empty(A, I, dtype=adt, device=dev)
    y = torch.empty(A, H, dtype=adt, device=dev)
    out = torch.empty(T, H, dtype=adt, device=dev)

    mx8 = args.path == "mx8"
    if mx8 and cfg.fmt != "mxfp4":
        print("--path mx8 runs the MXFP4 bank workload (--config mxfp4)", file=sys.stderr)
        sys.exit(2)
    if mx8:
        wsm = torch.empty(moeq.lib().mx8_workspace_bytes(A, max(H, I)), dtype=torch.uint8,
                          device=dev)

    def gate_up(w):
        if mx8:
            moeq.mx8_grouped_swiglu(route, bufs["values"], w["gate"], cfg.clamp, 1.0, 0.0,
                                    h=h, workspace=wsm)
        else:
            moeq.awq_grouped_swiglu(route, bufs["values"], w["gate"], w["up_arg"], cfg.clamp,
                                    1.0, 0.0, h)

    def step(i):
        w = replicas[i % R]
        moeq.moe_dispatch(base["x"], base["logits"], base["router_bias"], k, route, bufs)
        gate_up(w)
        if mx8:
            moeq.mx8_grouped_down(route, h, w["down"], y, workspace=wsm)
        else:
            moeq.awq_grouped_down(route, h, w["down"], y)
        moeq.moe_combine(route, y, bufs["weights"], out)

    if args.path == "unsorted":
        if cfg.fmt != "awq":
            print("the unsorted-row path is measured on AWQ cubes", file=sys.stderr)
            sys.exit(2)
        step(0)
        xr = base["x"].repeat_interleave(k, dim=0).contiguous()   # one row per assignment
        ids = bufs["selected"].view(-1).contiguous()               # token order, global IDs
        yu = torch.empty(A, I, dtype=adt, device=dev)
        wsu = torch.empty(moeq.awq_expert_workspace_bytes(A, E, H, I, adt), dtype=torch.uint8,
                          device=dev)
        for i in range(max(args.warmup, R)):
            moeq.awq_expert_forward(xr, ids, replicas[i % R]["gate"], yu, wsu)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            moeq.awq_expert_forward(xr, ids, replicas[i % R]["gate"], yu, wsu)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        ab = alg_bytes(p, route.expert_offsets.cpu().numpy())
        ub = ab["w_gateup"] // 2 + A * H * (2 if cfg.adt == "bf16" else 4) + \
            A * I * (2 if cfg.adt == "bf16" else 4)
        uf = 2 * A * H * I
        ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if uf / ub > ridge:
            bound, peak, unit, achieved = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s", uf / (ms * 1e-3) / 1e12
        else:
            bound, peak, unit, achieved = "hbm", HBM_PEAK_GBS, "GB/s", ub / (ms * 1e-3) / 1e9
        res = {
            "metric": METRIC_UNSORTED, "value": round(A / (ms * 1e-3), 1), "unit": "rows/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16" if cfg.adt == "bf16" else "f32", "data": "synthetic",
            "config": {"workload": workload_name(cfg), "rows": A, "touched_experts": ab["touched"],
                       "weight_replicas": R, "graph": False, "path": "unsorted"},
            "roofline": {"kernel": "awq_expert_forward (host ID check + sort + gather + "
                                   "grouped projection + restore), host clock",
                         "bound": bound, "achieved": round(achieved, 1), "peak": peak,
                         "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
                         "kernel_ms": round(ms, 5), "alg_bytes_per_launch": ub,
                         "alg_flops_per_launch": uf},
        }
        print(json.dumps(res), flush=True)
        return

    backward = args.path == "backward"
    if backward:
        if cfg.fmt != "awq":
            print("the backward chain is implemented for AWQ cubes", file=sys.stderr)
            sys.exit(2)
        step(0)   # the forward's values, y and routing, resident before timing
        gen = torch.Generator(device=dev).manual_seed(5)
        gout = torch.randn(T, H, generator=gen, device=dev).to(adt)
        gy = torch.empty(A, H, dtype=adt, device=dev)
        gw = torch.empty(T, k, dtype=torch.float32, device=dev)
        gv = torch.empty(A, H, dtype=adt, device=dev)
        gx = torch.empty(T, H, dtype=adt, device=dev)
        gl = torch.empty(T, E, dtype=torch.float32, device=dev)
        wsp = torch.empty(moeq.awq_swiglu_input_backward_workspace_bytes(A, I, adt),
                          dtype=torch.uint8, device=dev)

        def chain(w):
            moeq.awq_swiglu_input_backward(route, bufs["values"], w["gate"], w["up_arg"],
                                           w["down"], gy, cfg.clamp, 1.0, 0.0, wsp, gv)

        def step(i):  # noqa: F811 -- the backward step replaces the forward one
            w = replicas[i % R]
            moeq.moe_combine_backward(route, y, bufs["weights"], gout, grad_y=gy,
                                      grad_weights=gw)
            chain(w)
            moeq.moe_dispatch_backward(route, gv, gx)
            moeq.moe_dispatch_weights_backward(route, bufs["selected"], bufs["weights"], gw,
                                               gl)

    # warm-up (also before capture, on a side stream as graph capture expects)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(args.warmup, R)):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graphs = cycle = None
    if not args.eager:
        # one graph per replica, and one holding a whole cycle of R steps (the
        # way consecutive MoE layers of a model would be captured together)
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle):
            for r in range(R):
                step(r)
        for i in range(args.warmup):
            graphs[i % R].replay()
        cycle.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graphs is not None:
        full, rest = divmod(args.steps, R)
        for _ in range(full):
            cycle.replay()
        for i in range(rest):
            graphs[i].replay()
    else:
        for i in range(args.steps):
            step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # ---- dominant kernel (gate/up projection): per-launch HIP events on its stream
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i, (a, b) in enumerate(evs):
        w = replicas[i % R]
        a.record(stream)
        if backward:
            chain(w)
        else:
            gate_up(w)
        b.record(stream)
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    if backward:
        offsets = route.expert_offsets.cpu().numpy()
        ab = alg_bytes(p, offsets)
        cb = bwd_alg_bytes(p, ab)
        cf = 10 * A * H * I   # down VJP, gate/up recompute, two transposed products
        ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if cf / cb > ridge:
            bound, peak, unit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
            achieved = cf / (k_ms * 1e-3) / 1e12
        else:
            bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
            achieved = cb / (k_ms * 1e-3) / 1e9
        res = {
            "metric": METRIC_BWD, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if cfg.adt == "bf16" else "f32",
            "data": "synthetic",
            "config": {"workload": workload_name(cfg), "tokens": T, "assignments": A,
                       "touched_experts": ab["touched"], "weight_replicas": R,
                       "graph": graphs is not None, "path": "backward"},
            "roofline": {"kernel": "awq_swiglu_input_backward (down VJP + gate/up recompute "
                                   "with SwiGLU VJP + transposed gate/up)",
                         "bound": bound, "achieved": round(achieved, 1), "peak": peak,
                         "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
                         "kernel_ms": round(k_ms, 5), "alg_bytes_per_launch": cb,
                         "alg_flops_per_launch": cf},
        }
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_backward(cfg, args.cpu_seconds)
        print(json.dumps(res), flush=True)
        return

    offsets = route.expert_offsets.cpu().numpy()
    ab = alg_bytes(p, offsets)
    F = flops(p)
    tok_s = T / (ms * 1e-3)
    # the gate/up call's own bound: MFMA above the ridge point, else HBM
    gu_flops = 4 * A * p["H"] * p["I"]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mx8:   # the fp8 x fp4 block-scaled MFMA: against the dense fp8 peak
        bound, peak, unit = "mfma", FP8_PEAK_TFLOPS, "TFLOP/s"
        achieved = gu_flops / (k_ms * 1e-3) / 1e12
    elif gu_flops / ab["gateup"] > ridge:
        bound, peak, unit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
        achieved = gu_flops / (k_ms * 1e-3) / 1e12
    else:
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        achieved = ab["gateup"] / (k_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg.name)
    path_gbs = ab["total"] / (ms * 1e-3) / 1e9
    path_tflops = F / (ms * 1e-3) / 1e12
    res = {
        "metric": METRIC_MX8 if mx8 else METRIC, "value": round(tok_s, 1), "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8xmxfp4" if mx8 else ("bf16" if cfg.adt == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "tokens": T, "assignments": A,
                   "touched_experts": ab["touched"], "weight_replicas": R,
                   "graph": graphs is not None},
        "roofline": {"kernel": ("mx8_grouped_swiglu (MXFP8 quantization + block-scaled "
                                "MFMA gate/up + SwiGLU)") if mx8 else
                               "awq_grouped_swiglu (gate/up dequant-GEMM + SwiGLU)",
                     "bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel_ms": round(k_ms, 5),
                     "alg_bytes_per_launch": ab["gateup"], "alg_flops_per_launch": gu_flops},
        "path": {"alg_bytes": ab["total"], "alg_flops": F, "GBs": round(path_gbs, 1),
                 "hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
                 "TFLOPs": round(path_tflops, 2),
                 "mfma_frac": round(path_tflops / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
