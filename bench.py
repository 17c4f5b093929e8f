"""Benchmark: MoE expert-FFN tokens/s on one MI355X, with the roofline of the
dominant kernel and the CPU oracle timed beside it.

One step = the whole forward path over one batch: moe_dispatch (router top-k +
softmax + stable COPY dispatch) -> awq_grouped_swiglu -> awq_grouped_down ->
moe_combine.  Inputs are seeded synthetic tensors resident in HBM before the
timed region.  Each step reads a different replica of the expert weights (as
consecutive MoE layers would), so no step finds the previous step's weights in
the 256 MB last-level cache.  Steps are captured once as HIP graphs -- a whole
cycle over the replicas in one graph -- and replayed.

Prints ONE JSON line.  `value` is the decode-shaped AWQ MoE (T=64, hidden 2048,
intermediate 768, 128 experts, top_k 8, group 128, bf16); the same line carries
the prefill-shaped, many-expert and MXFP4-bank workloads under "workloads"
(--single measures only --config).

Per-call times come from HIP graphs of back-to-back launches of that one call
(cycling the weight replicas), timed with HIP events on the stream the graph is
replayed on, divided by the launch count: the kernels' own time plus the gap
between graph nodes, as a kernel trace sees it.  `roofline` is the gate/up call.

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

--summarize-stats / --summarize-traffic turn rocprofv3 CSV output into the text
summaries kept under profiles/ (see their headers for the commands).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA (the fp8 x fp4 scaled MFMA's operand type)
METRIC = "MoE expert-FFN tokens/s at 1 GPU; % of HBM (decode) / MFMA (prefill) peak"
METRIC_BWD = "MoE expert-FFN backward tokens/s at 1 GPU (first-order input VJPs)"
METRIC_MX8 = "MoE expert-FFN tokens/s at 1 GPU, MXFP4 bank on the block-scaled MFMA (MXFP8 activations)"
METRIC_UNSORTED = "unsorted-row expert projection rows/s at 1 GPU (gate cube, rows in token order)"
OTHER_WORKLOADS = ("prefill", "many", "mxfp4")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="after the warm-up steps, untimed replays of the step graphs for at "
                         "least this long, so the timed steps start at steady clocks")
    ap.add_argument("--config", default="decode",
                    choices=["tiny", "decode", "prefill", "many", "mxfp4"])
    ap.add_argument("--single", action="store_true",
                    help="measure only --config (no other workloads in the line)")
    ap.add_argument("--replica-bytes", type=float, default=1.2e9,
                    help="weight bytes cycled through by consecutive steps")
    ap.add_argument("--path", default="forward",
                    choices=["forward", "backward", "unsorted", "mx8"])
    ap.add_argument("--eager", action="store_true", help="no HIP graph capture")
    ap.add_argument("--kernel-launches", type=int, default=0,
                    help="launches per kernel-timing graph (default: replicas x ceil(16/R))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA and HBM peaks")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 launches): the "
                         "known-size reference that scales the HBM byte counters")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a summary of rocprofv3 --stats output found under DIR")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="print the HBM traffic summary of the gate/up kernel from four "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, and the same over "
                         "a plain copy)")
    ap.add_argument("--kernel", default="",
                    help="kernel-name substring for --summarize-traffic")
    ap.add_argument("--title", default="", help="header line for the summaries")
    ap.add_argument("--tail", type=int, default=0,
                    help="--summarize-stats: also average each kernel's last TAIL dispatches")
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
    dispatch = T * E * 4 + T * H * ab + A * H * ab + T * k * 4   # logits, x, values, weights
    combine = A * H * ab + T * k * 4 + T * H * ab                 # y, weights, out
    return dict(touched=touched, gateup=w_gu + act_gu, down=w_dn + act_dn,
                dispatch=dispatch, combine=combine,
                total=w_gu + w_dn + act_gu + act_dn + dispatch + combine,
                weights=w_gu + w_dn, w_gateup=w_gu, w_down=w_dn)


def flops(p):
    A = p["T"] * p["k"]
    return 6 * A * p["H"] * p["I"]


def roofline(name, nbytes, nflops, ms, peak_tflops=BF16_PEAK_TFLOPS):
    """Bound by arithmetic intensity against the ridge point of the dtype's peak."""
    ridge = peak_tflops * 1e12 / (HBM_PEAK_GBS * 1e9)
    if nflops / nbytes > ridge:
        bound, peak, unit, ach = "mfma", peak_tflops, "TFLOP/s", nflops / (ms * 1e-3) / 1e12
    else:
        bound, peak, unit, ach = "hbm", HBM_PEAK_GBS, "GB/s", nbytes / (ms * 1e-3) / 1e9
    return {"kernel": name, "bound": bound, "achieved": round(ach, 1), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4), "kernel_ms": round(ms, 5),
            "alg_bytes_per_launch": int(nbytes), "alg_flops_per_launch": int(nflops)}


def source_digest():
    """Digest of every kernel source of the library (a counter summary taken on
    other sources is not reported)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_moe_expert_router_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*.hip")) +
                       glob.glob(os.path.join(csrc, "*.hpp")) +
                       glob.glob(os.path.join(csrc, "*.cpp"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config_name):
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counters), or
    None when there is none for this workload or the sources changed since."""
    path = os.path.join(ROOT, "profiles", f"gate_up.{config_name}.traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_digest") != source_digest():
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_cores():
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))


def cpu_baseline(cfg, target_s):
    """The oracle as it stands, on a bounded sample of the same workload."""
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
    return {"value": round(reps * T / el, 3), "unit": "tokens/s", "cores": cpu_cores(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{reps} x full forward of a {T}-token batch of this workload "
                      f"({el:.1f} s, double accumulation, OpenMP)"}


def cpu_single_core(target_s):
    """Single-core figures of the oracle (one OpenMP thread) for the tiny
    workload and a 4-token sample of the decode workload."""
    import ctypes
    import oracle
    from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs
    oracle._load()
    gomp = ctypes.CDLL("libgomp.so.1")  # the oracle's OpenMP runtime, already loaded
    prev = gomp.omp_get_max_threads()
    gomp.omp_set_num_threads(1)
    out = {}
    try:
        for name, T in (("tiny", 16), ("decode", 4)):
            p = make_inputs(CONFIGS[name], T=T)
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.moe_forward(p, keep_intermediates=False)
                reps += 1
                el = time.perf_counter() - t0
                if el >= target_s or reps >= 1000:
                    break
            out[name] = {"value": round(reps * T / el, 3), "unit": "tokens/s", "cores": 1,
                         "sample": f"{reps} x full forward of a {T}-token batch ({el:.1f} s)"}
    finally:
        gomp.omp_set_num_threads(prev)
    return out


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
    return {"value": round(reps * T / el, 3), "unit": "tokens/s", "cores": cpu_cores(),
            "cpu": cpu_model(), "kind": "oracle",
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


class Workload:
    """Inputs, weight replicas and output buffers of one workload, on cuda:0."""

    def __init__(self, cfg, replica_bytes, mx8=False):
        import torch

        from quantized_moe_expert_router_amd import device_inputs as di
        from quantized_moe_expert_router_amd import moeq
        from quantized_moe_expert_router_amd.synth import make_inputs, weight_bytes
        self.torch, self.moeq = torch, moeq
        self.cfg, self.mx8 = cfg, mx8
        self.dev = dev = torch.device("cuda:0")
        self.p = p = make_inputs(cfg)
        self.base = base = di.upload(p, dev)
        self.R = R = max(2, math.ceil(replica_bytes / weight_bytes(p)))
        wkeys = ("gate", "up_arg", "down")

        def clone(w):
            if w is None:
                return None
            if isinstance(w, moeq.AwqExperts):
                return moeq.AwqExperts(w.qweight.clone(), w.qzeros.clone(), w.scales.clone(),
                                       w.group_size, None if w.bias is None else w.bias.clone())
            return moeq.Mxfp4Bank(w.blocks.clone(), w.scales.clone(), w.bias.clone(),
                                  w.interleaved_gate_up)
        self.replicas = [{k: base[k] for k in wkeys}] + [{k: clone(base[k]) for k in wkeys}
                                                         for _ in range(R - 1)]
        T, k, H, I, E = cfg.T, cfg.k, cfg.H, cfg.I, cfg.E
        self.A = A = T * k
        adt = base["x"].dtype
        self.route = moeq.RouteState(T, E, k, dev)
        self.bufs = dict(values=torch.empty(A, H, dtype=adt, device=dev),
                         weights=torch.empty(T, k, dtype=torch.float32, device=dev),
                         selected=torch.empty(T, k, dtype=torch.int32, device=dev),
                         row_experts=torch.empty(A, dtype=torch.int32, device=dev))
        self.h = torch.empty(A, I, dtype=adt, device=dev)
        self.y = torch.empty(A, H, dtype=adt, device=dev)
        self.out = torch.empty(T, H, dtype=adt, device=dev)
        self.wsm = None
        if mx8:
            self.wsm = torch.empty(moeq.lib().mx8_workspace_bytes(A, max(H, I)),
                                   dtype=torch.uint8, device=dev)

    # the four calls of one forward step
    def dispatch(self, i=0):
        b = self.base
        self.moeq.moe_dispatch(b["x"], b["logits"], b["router_bias"], self.cfg.k, self.route,
                               self.bufs)

    def gate_up(self, i=0):
        w, c = self.replicas[i % self.R], self.cfg
        if self.mx8:
            self.moeq.mx8_grouped_swiglu(self.route, self.bufs["values"], w["gate"], c.clamp,
                                         1.0, 0.0, h=self.h, workspace=self.wsm)
        else:
            self.moeq.awq_grouped_swiglu(self.route, self.bufs["values"], w["gate"],
                                         w["up_arg"], c.clamp, 1.0, 0.0, self.h)

    def down(self, i=0):
        w = self.replicas[i % self.R]
        if self.mx8:
            self.moeq.mx8_grouped_down(self.route, self.h, w["down"], self.y,
                                       workspace=self.wsm)
        else:
            self.moeq.awq_grouped_down(self.route, self.h, w["down"], self.y)

    def combine(self, i=0):
        self.moeq.moe_combine(self.route, self.y, self.bufs["weights"], self.out)

    def step(self, i):
        self.dispatch(i)
        self.gate_up(i)
        self.down(i)
        self.combine(i)


SETTLE_MS = 200.0  # set from --settle-ms


def settle(torch, replay):
    """Untimed replays until SETTLE_MS of wall time has passed: with a few warm-up
    steps only, the first steps after a phase of other work run 5-10% slower
    (the GPU clocks ramp), and a timed region of 20 decode steps is under 2 ms."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(8):
            replay()
        torch.cuda.synchronize()


def warm_and_capture(torch, step, R, warmup, eager):
    """Warm-up on a side stream, then one graph per replica and one graph of a
    whole cycle of R steps (as consecutive MoE layers of a model would be), then
    untimed replays of the cycle for SETTLE_MS."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(warmup, R)):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    if eager:
        it = iter(range(1 << 30))
        settle(torch, lambda: step(next(it)))
        return None, None
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
    for i in range(warmup):
        graphs[i % R].replay()
    cycle.replay()
    torch.cuda.synchronize()
    settle(torch, cycle.replay)
    return graphs, cycle


def timed_steps(torch, steps, R, graphs, cycle, step):
    """Exactly `steps` steps between two events (synchronised on both sides):
    mean ms per step."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graphs is not None:
        full, rest = divmod(steps, R)
        for _ in range(full):
            cycle.replay()
        for i in range(rest):
            graphs[i].replay()
    else:
        for i in range(steps):
            step(i)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def median_step(torch, steps, R, graphs):
    """Median of per-replay event pairs over single-step graphs (outside the
    timed region)."""
    import numpy as np
    if graphs is None:
        return None
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        graphs[i % R].replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def call_ms(torch, launch, R, launches):
    """Per-launch time of one call: a graph of `launches` back-to-back launches
    (replica i % R for launch i), replayed and timed with events on the stream
    it is replayed on, divided by the launch count.  Three untimed replays
    first, then the median of three timed rounds of five replays: the first
    replays after the other calls' timing run slower (the GFX clock settles),
    and a single round caught that transient."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(R):
            launch(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(launches):
            launch(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    reps, rounds = 5, []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        rounds.append(a.elapsed_time(b) / (reps * launches))
    return sorted(rounds)[1]


def measure_forward(cfg, args, steps, warmup, mx8=False):
    """One workload's forward step: timed steps, median step, per-call times and
    rooflines."""
    import torch
    wl = Workload(cfg, args.replica_bytes, mx8=mx8)
    p, R, A = wl.p, wl.R, wl.A
    graphs, cycle = warm_and_capture(torch, wl.step, R, warmup, args.eager)
    ms = timed_steps(torch, steps, R, graphs, cycle, wl.step)
    med = median_step(torch, steps, R, graphs)
    launches = args.kernel_launches or R * math.ceil(16 / R)
    calls = {nm: call_ms(torch, getattr(wl, nm), R, launches)
             for nm in ("dispatch", "gate_up", "down", "combine")}
    wl.step(0)
    torch.cuda.synchronize()
    offsets = wl.route.expert_offsets.cpu().numpy()
    ab = alg_bytes(p, offsets)
    H, I = p["H"], p["I"]
    peak = FP8_PEAK_TFLOPS if mx8 else BF16_PEAK_TFLOPS
    gu_name = ("mx8_grouped_swiglu (MXFP8 quantization + block-scaled MFMA gate/up + SwiGLU)"
               if mx8 else "awq_grouped_swiglu (gate/up dequant-GEMM + SwiGLU)")
    dn_name = ("mx8_grouped_down (MXFP8 quantization + block-scaled MFMA down)" if mx8
               else "awq_grouped_down (down dequant-GEMM)")
    rl_gu = roofline(gu_name, ab["gateup"], 4 * A * H * I, calls["gate_up"], peak)
    rl_gu["traffic"] = None if mx8 else measured_traffic(cfg.name)
    rl_dn = roofline(dn_name, ab["down"], 2 * A * H * I, calls["down"], peak)
    F = flops(p)
    path_gbs = ab["total"] / (ms * 1e-3) / 1e9
    path_tflops = F / (ms * 1e-3) / 1e12
    return dict(
        cfg=cfg, wl=wl, ms=ms, median_ms=med, R=R, ab=ab, roofline=rl_gu,
        result={
            "workload": workload_name(cfg), "tokens": cfg.T, "assignments": A,
            "touched_experts": ab["touched"], "ms_per_step": round(ms, 5),
            "median_ms_per_step": None if med is None else round(med, 5),
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "calls_us": {k: round(v * 1e3, 2) for k, v in calls.items()},
            "calls_sum_ms": round(sum(calls.values()), 5),
            "roofline_gate_up": rl_gu, "roofline_down": rl_dn,
            "path": {"alg_bytes": ab["total"], "alg_flops": F, "GBs": round(path_gbs, 1),
                     "hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
                     "TFLOPs": round(path_tflops, 2),
                     "mfma_frac": round(path_tflops / BF16_PEAK_TFLOPS, 4)},
        })


def measured_peaks():
    """Peaks measured on this GPU beside the published ones: a dense bf16 MFMA
    loop on register operands (both MFMA shapes, 1, 2 and 4 waves per SIMD, the
    best), a streaming HBM read of 4 GiB, and a 1 GiB device copy (read + write)."""
    import ctypes as C
    import torch
    lib = C.CDLL(os.path.join(ROOT, "quantized_moe_expert_router_amd", "csrc",
                              "libmoeq_peaks.so"))
    lib.moeq_peak_mfma_bf16.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                        C.c_void_p]
    lib.moeq_peak_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_void_p]
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        return best

    res = {}
    blocks, iters = 256 * 4, 200
    out = torch.empty(blocks * 64 * 16, dtype=torch.float32, device="cuda:0")
    for shape, flop in ((0, 16384), (1, 32768)):
        best = 0.0
        for waves in (4, 8, 16):
            def run():
                rc = lib.moeq_peak_mfma_bf16(blocks, waves, iters, shape,
                                             C.c_void_p(out.data_ptr()), sp)
                assert rc == 0, rc
            t = timed(run)
            best = max(best, blocks * waves * iters * 8 * flop / t / 1e12)
        res["mfma_bf16_16x16x32_tflops" if shape == 0 else "mfma_bf16_32x32x16_tflops"] = round(best, 1)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    rblocks = 256 * 8
    rout = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda:0")

    def read():
        rc = lib.moeq_peak_read(C.c_void_p(buf.data_ptr()), nbytes, rblocks,
                                C.c_void_p(rout.data_ptr()), sp)
        assert rc == 0, rc
    res["hbm_read_gbs"] = round(nbytes / timed(read) / 1e9, 1)
    half = buf[: 1 << 30]
    dst = buf[1 << 30: 2 << 30]
    res["hbm_copy_gbs"] = round(2 * (1 << 30) / timed(lambda: dst.copy_(half)) / 1e9, 1)
    del buf, out, rout
    torch.cuda.empty_cache()
    res["method"] = ("best of 3 HIP-event-timed launches; MFMA: 1024 blocks x 4/8/16 waves, "
                     "200 x 8 MFMAs per wave on registers; read: 4 GiB by 2048 blocks, "
                     "16-byte loads; copy: torch 1 GiB device copy, bytes read + written")
    return res


def with_measured(rl, peaks):
    """Add the fraction of the measured peak of the same kind to a roofline."""
    if not peaks:
        return rl
    if rl["bound"] == "hbm":
        ref = peaks["hbm_read_gbs"]
    elif rl["peak"] == BF16_PEAK_TFLOPS:
        ref = max(peaks["mfma_bf16_16x16x32_tflops"], peaks["mfma_bf16_32x32x16_tflops"])
    else:
        return rl
    rl["measured_peak"] = ref
    rl["frac_of_measured"] = round(rl["achieved"] / ref, 4)
    return rl


def release(torch, m):
    m.pop("wl", None)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_unsorted(cfg, args):
    import torch
    from quantized_moe_expert_router_amd import moeq
    if cfg.fmt != "awq":
        print("the unsorted-row path is measured on AWQ cubes", file=sys.stderr)
        sys.exit(2)
    wl = Workload(cfg, args.replica_bytes)
    p, R, A = wl.p, wl.R, wl.A
    H, I, E, k = cfg.H, cfg.I, cfg.E, cfg.k
    adt = wl.base["x"].dtype
    wl.step(0)
    xr = wl.base["x"].repeat_interleave(k, dim=0).contiguous()   # one row per assignment
    ids = wl.bufs["selected"].view(-1).contiguous()               # token order, global IDs
    yu = torch.empty(A, I, dtype=adt, device=wl.dev)
    wsu = torch.empty(moeq.awq_expert_workspace_bytes(A, E, H, I, adt), dtype=torch.uint8,
                      device=wl.dev)
    for i in range(max(args.warmup, R)):
        moeq.awq_expert_forward(xr, ids, wl.replicas[i % R]["gate"], yu, wsu)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        moeq.awq_expert_forward(xr, ids, wl.replicas[i % R]["gate"], yu, wsu)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ab = alg_bytes(p, wl.route.expert_offsets.cpu().numpy())
    ab_el = 2 if cfg.adt == "bf16" else 4
    ub = ab["w_gateup"] // 2 + A * H * ab_el + A * I * ab_el
    rl = roofline("awq_expert_forward (host ID check + sort + gather + grouped projection + "
                  "restore), host clock", ub, 2 * A * H * I, ms)
    rl["traffic"] = None
    return {
        "metric": METRIC_UNSORTED, "value": round(A / (ms * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.adt == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": workload_name(cfg), "rows": A, "touched_experts": ab["touched"],
                   "weight_replicas": R, "graph": False, "path": "unsorted"},
        "roofline": rl,
    }


def run_backward(cfg, args):
    import torch
    from quantized_moe_expert_router_amd import moeq
    if cfg.fmt != "awq":
        print("the backward chain is implemented for AWQ cubes", file=sys.stderr)
        sys.exit(2)
    wl = Workload(cfg, args.replica_bytes)
    p, R, A = wl.p, wl.R, wl.A
    T, k, H, I, E = cfg.T, cfg.k, cfg.H, cfg.I, cfg.E
    adt, dev = wl.base["x"].dtype, wl.dev
    wl.step(0)   # the forward's values, y and routing, resident before timing
    gen = torch.Generator(device=dev).manual_seed(5)
    gout = torch.randn(T, H, generator=gen, device=dev).to(adt)
    gy = torch.empty(A, H, dtype=adt, device=dev)
    gw = torch.empty(T, k, dtype=torch.float32, device=dev)
    gv = torch.empty(A, H, dtype=adt, device=dev)
    gx = torch.empty(T, H, dtype=adt, device=dev)
    gl = torch.empty(T, E, dtype=torch.float32, device=dev)
    wsp = torch.empty(moeq.awq_swiglu_input_backward_workspace_bytes(A, I, adt),
                      dtype=torch.uint8, device=dev)
    route, bufs = wl.route, wl.bufs

    def chain(i):
        w = wl.replicas[i % R]
        moeq.awq_swiglu_input_backward(route, bufs["values"], w["gate"], w["up_arg"],
                                       w["down"], gy, cfg.clamp, 1.0, 0.0, wsp, gv)

    def step(i):
        moeq.moe_combine_backward(route, wl.y, bufs["weights"], gout, grad_y=gy,
                                  grad_weights=gw)
        chain(i)
        moeq.moe_dispatch_backward(route, gv, gx)
        moeq.moe_dispatch_weights_backward(route, bufs["selected"], bufs["weights"], gw, gl)

    graphs, cycle = warm_and_capture(torch, step, R, args.warmup, args.eager)
    ms = timed_steps(torch, args.steps, R, graphs, cycle, step)
    med = median_step(torch, args.steps, R, graphs)
    k_ms = call_ms(torch, chain, R, args.kernel_launches or R * math.ceil(16 / R))
    ab = alg_bytes(p, route.expert_offsets.cpu().numpy())
    rl = roofline("awq_swiglu_input_backward (down VJP + gate/up recompute with SwiGLU VJP + "
                  "transposed gate/up)", bwd_alg_bytes(p, ab), 10 * A * H * I, k_ms)
    rl["traffic"] = None
    res = {
        "metric": METRIC_BWD, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.adt == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "tokens": T, "assignments": A,
                   "touched_experts": ab["touched"], "weight_replicas": R,
                   "graph": graphs is not None, "path": "backward"},
        "roofline": rl,
        "median_ms_per_step": None if med is None else round(med, 5),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(cfg, args.cpu_seconds)
    return res


# ------------------------------------------------------------------ profile summaries
def _csvs(d, name):
    return sorted(glob.glob(os.path.join(d, "**", name), recursive=True))


def summarize_stats(d, title, tail=0):
    """Kernel statistics table from rocprofv3 --stats output under d."""
    files = _csvs(d, "*kernel_stats.csv")
    if not files:
        sys.exit(f"no *kernel_stats.csv under {d}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    rows.sort(key=lambda r: -r[5])
    if title:
        print(f"# {title}")
    print(f"# source: {os.path.relpath(files[0], ROOT)}")
    print(f"\n{'kernel':100s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for name, calls, avg, mn, mx, pct in rows:
        print(f"{name[:100]:100s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {pct:6.2f}")
    traces = _csvs(d, "*kernel_trace.csv")
    if tail and traces:
        # the last `tail` dispatches of each kernel: the timed replays of the
        # per-call timing graphs, which bench.py runs last for every call
        per = {}
        with open(traces[0]) as f:
            for r in csv.DictReader(f):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        print(f"\n# last {tail} dispatches of each kernel (the per-call timing graphs' timed "
              "replays)")
        print(f"{'kernel':100s} {'calls':>6s} {'avg_us':>9s}")
        for name, ev in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
            ev.sort()
            last = [d for _, d in ev[-tail:]]
            if len(ev) >= tail:
                print(f"{name[:100]:100s} {len(last):6d} {sum(last) / len(last) / 1e3:9.2f}")
    if traces:
        # each dispatch by the kernel that ran before it: after another kernel (as
        # inside the forward step) or after itself (the per-call timing graphs'
        # back-to-back launches)
        seq = []
        with open(traces[0]) as f:
            for r in csv.DictReader(f):
                seq.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
        seq.sort()
        ctx = {}
        for (_, _, prev), (s0, e0, name) in zip(seq, seq[1:]):
            ctx.setdefault(name, ([], []))[prev == name].append((e0 - s0) / 1e3)
        med = lambda v: sorted(v)[len(v) // 2] if v else float("nan")
        print("\n# median duration by the preceding dispatch: another kernel (in the step) or "
              "the same kernel (back to back)")
        print(f"{'kernel':100s} {'n_step':>6s} {'step_us':>9s} {'n_b2b':>6s} {'b2b_us':>9s}")
        for name, (other, same) in sorted(ctx.items(), key=lambda kv: -sum(kv[1][0] + kv[1][1])):
            if len(other) + len(same) >= 16:
                print(f"{name[:100]:100s} {len(other):6d} {med(other):9.2f} {len(same):6d} "
                      f"{med(same):9.2f}")


def _counter_per_dispatch(d, counter, kernel_sub):
    """Mean over matching dispatches of one counter (summed over its instances)."""
    files = _csvs(d, "*counter_collection.csv")
    if not files:
        sys.exit(f"no *counter_collection.csv under {d}")
    per = {}
    names = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or kernel_sub not in r["Kernel_Name"]:
                continue
            key = r["Dispatch_Id"]
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    if not per:
        sys.exit(f"no {counter} dispatches of '{kernel_sub}' under {d}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals), sorted(set(names.values()))


def summarize_traffic(dirs, kernel_sub, title, alg_bytes_per_launch=None):
    """kernel_sub: one name substring, or several separated by '|' for a call
    made of several kernels (their per-dispatch means add up)."""
    fetch = write = 0.0
    names, nf, nw = [], 0, 0
    for sub in kernel_sub.split("|"):
        f1, n1, nm1 = _counter_per_dispatch(dirs[0], "FETCH_SIZE", sub)
        w1, n2, _ = _counter_per_dispatch(dirs[1], "WRITE_SIZE", sub)
        fetch, write, nf, nw = fetch + f1, write + w1, nf + n1, nw + n2
        names += nm1
    cf, _, _ = _counter_per_dispatch(dirs[2], "FETCH_SIZE", "copyBuffer")
    cw, _, _ = _counter_per_dispatch(dirs[3], "WRITE_SIZE", "copyBuffer")
    copy_bytes = 1 << 30      # bench.py --copy-probe-mib 1024: 1 GiB read and 1 GiB written
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    traffic = fetch * 1024 * ff + write * 1024 * wf
    if title:
        print(f"# {title}")
    print("# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; the factors scale them by what the")
    print(f"# same counters read for a plain copy of {copy_bytes} bytes each way.")
    for nm in names:
        print(f"kernel: {nm[:160]}")
    print(f"dispatches_fetch: {nf}")
    print(f"dispatches_write: {nw}")
    print(f"fetch_kib_per_dispatch: {fetch:.1f}")
    print(f"write_kib_per_dispatch: {write:.1f}")
    print(f"copy_fetch_kib_per_dispatch: {cf:.1f}")
    print(f"copy_write_kib_per_dispatch: {cw:.1f}")
    print(f"fetch_factor: {ff:.4f}")
    print(f"write_factor: {wf:.4f}")
    print(f"traffic_bytes_per_launch: {traffic:.0f}")
    if alg_bytes_per_launch:
        print(f"algorithmic_bytes_per_launch: {alg_bytes_per_launch}")
        print(f"traffic_over_algorithmic: {traffic / alg_bytes_per_launch:.4f}")
    print(f"source_digest: {source_digest()}")


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = max(0.0, args.settle_ms)
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.title, args.tail)
        return
    if args.summarize_traffic:
        alg = None
        if args.config:
            from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs
            import numpy as np
            import oracle
            p = make_inputs(CONFIGS[args.config])
            sel, _ = oracle.route(p["logits"], p["router_bias"], p["k"])
            off, _, _, _ = oracle.dispatch_index(sel, p["E"])
            alg = alg_bytes(p, off)["gateup"]
        summarize_traffic(args.summarize_traffic, args.kernel, args.title, alg)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path "
              "would shard by tokens or by expert ranges across GPUs)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return

    import torch

    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd.synth import CONFIGS

    cfg = CONFIGS[args.config]
    torch.cuda.set_device(0)
    moeq.lib()
    if args.path == "unsorted":
        print(json.dumps(run_unsorted(cfg, args)), flush=True)
        return
    if args.path == "backward":
        print(json.dumps(run_backward(cfg, args)), flush=True)
        return
    mx8 = args.path == "mx8"
    if mx8 and cfg.fmt != "mxfp4":
        print("--path mx8 runs the MXFP4 bank workload (--config mxfp4)", file=sys.stderr)
        sys.exit(2)

    peaks = None if args.no_peaks else measured_peaks()
    head = measure_forward(cfg, args, args.steps, args.warmup, mx8=mx8)
    r = head["result"]
    with_measured(head["roofline"], peaks)
    with_measured(r["roofline_down"], peaks)
    res = {
        "metric": METRIC_MX8 if mx8 else METRIC, "value": r["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": SETTLE_MS, "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8xmxfp4" if mx8 else ("bf16" if cfg.adt == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": r["workload"], "tokens": cfg.T, "assignments": head["wl"].A,
                   "touched_experts": r["touched_experts"], "weight_replicas": head["R"],
                   "graph": not args.eager},
        "roofline": head["roofline"],
        "median_ms_per_step": r["median_ms_per_step"],
        "calls_us": r["calls_us"],
        "roofline_down": r["roofline_down"],
        "path": r["path"],
    }
    release(torch, head)
    if not args.single and not mx8 and cfg.name == "decode":
        others = {}
        for name in OTHER_WORKLOADS:
            m = measure_forward(CONFIGS[name], args, min(args.steps, 100),
                                min(args.warmup, 10))
            others[name] = m["result"]
            with_measured(others[name]["roofline_gate_up"], peaks)
            with_measured(others[name]["roofline_down"], peaks)
            release(torch, m)
        res["workloads"] = others
    if peaks:
        res["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, args.cpu_seconds)
        cb["gpu_over_cpu"] = round(res["value"] / cb["value"], 1) if cb["value"] else None
        if not args.single and not mx8 and cfg.name == "decode":
            cb["single_core"] = cpu_single_core(min(args.cpu_seconds, 4.0))
            for name, w in res.get("workloads", {}).items():
                wb = cpu_baseline(CONFIGS[name], min(args.cpu_seconds, 5.0))
                wb["gpu_over_cpu"] = (round(w["tokens_per_s"] / wb["value"], 1)
                                      if wb["value"] else None)
                w["cpu_baseline"] = wb
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
