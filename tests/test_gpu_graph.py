"""Graph replays of the routed path against eager runs, through the C-ABI.

The forward calls (moe_dispatch, awq_grouped_swiglu, awq_grouped_down,
moe_combine) and, for AWQ cubes, the backward calls after them are captured
once in a HIP graph over fixed buffers.  Each replay runs on new token rows,
router logits and output gradients copied into the captured input buffers,
with eager work and synchronisations between the replays.  Every output of
every replay must equal an eager run on the same inputs bit for bit: the
kernels are deterministic (fixed summation orders, no atomics in any sum), and
no launch takes its grid from the routing, so one capture serves any routing.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import CONFIGS, make_inputs, to_storage

pytestmark = pytest.mark.gpu


class Step:
    """Fixed buffers for one configuration and the calls of one step."""

    def __init__(self, p, d, backward, mx8=False):
        T, k, E, H, I = p["T"], p["k"], p["E"], p["H"], p["I"]
        A = T * k
        adt = d["x"].dtype
        self.p, self.d, self.backward, self.mx8 = p, d, backward, mx8
        self.route = moeq.RouteState(T, E, k, torch.device(DEV))
        self.bufs = dict(values=torch.empty(A, H, dtype=adt, device=DEV),
                         weights=torch.empty(T, k, dtype=torch.float32, device=DEV),
                         selected=torch.empty(T, k, dtype=torch.int32, device=DEV),
                         row_experts=torch.empty(A, dtype=torch.int32, device=DEV))
        self.h = torch.empty(A, I, dtype=adt, device=DEV)
        self.y = torch.empty(A, H, dtype=adt, device=DEV)
        self.out = torch.empty(T, H, dtype=adt, device=DEV)
        if mx8:
            wsb = moeq.lib().mx8_workspace_bytes(A, max(H, I))
            self.wsm = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        if backward:
            self.gout = torch.zeros(T, H, dtype=adt, device=DEV)
            self.gy = torch.empty(A, H, dtype=adt, device=DEV)
            self.gw = torch.empty(T, k, dtype=torch.float32, device=DEV)
            self.gv = torch.empty(A, H, dtype=adt, device=DEV)
            self.gx = torch.empty(T, H, dtype=adt, device=DEV)
            self.gl = torch.empty(T, E, dtype=torch.float32, device=DEV)
            wsb = moeq.awq_swiglu_input_backward_workspace_bytes(A, I, adt)
            self.ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)

    def run(self):
        p, d, r = self.p, self.d, self.route
        moeq.moe_dispatch(d["x"], d["logits"], d["router_bias"], p["k"], r, self.bufs)
        if self.mx8:
            moeq.mx8_grouped_swiglu(r, self.bufs["values"], d["gate"], p["clamp"], p["alpha"],
                                    p["up_offset"], h=self.h, workspace=self.wsm)
            moeq.mx8_grouped_down(r, self.h, d["down"], self.y, workspace=self.wsm)
        else:
            moeq.awq_grouped_swiglu(r, self.bufs["values"], d["gate"], d["up_arg"], p["clamp"],
                                    p["alpha"], p["up_offset"], self.h)
            moeq.awq_grouped_down(r, self.h, d["down"], self.y)
        moeq.moe_combine(r, self.y, self.bufs["weights"], self.out)
        if self.backward:
            moeq.moe_combine_backward(r, self.y, self.bufs["weights"], self.gout,
                                      grad_y=self.gy, grad_weights=self.gw)
            moeq.awq_swiglu_input_backward(r, self.bufs["values"], d["gate"], d["up_arg"],
                                           d["down"], self.gy, p["clamp"], p["alpha"],
                                           p["up_offset"], self.ws, self.gv)
            moeq.moe_dispatch_backward(r, self.gv, self.gx)
            moeq.moe_dispatch_weights_backward(r, self.bufs["selected"], self.bufs["weights"],
                                               self.gw, self.gl)

    def outputs(self):
        r = self.route
        t = dict(self.bufs, h=self.h, y=self.y, out=self.out, offsets=r.expert_offsets,
                 row_src=r.row_src, slot_pos=r.slot_pos)
        if self.backward:
            t.update(gy=self.gy, gw=self.gw, gv=self.gv, gx=self.gx, gl=self.gl)
        return {k: v.detach().cpu().clone() for k, v in t.items() if isinstance(v, torch.Tensor)}


@pytest.mark.parametrize("name,T,backward,mx8", [
    ("tiny", 16, True, False),        # fp32 activations: generic kernels
    ("decode", 64, True, False),      # fused small dispatch, stream kernels
    ("prefill", 1024, True, False),   # four-launch dispatch, register-decoded MFMA kernels
    ("many", 1024, True, False),      # fp32 scales: warp-specialised MFMA kernels
    ("mxfp4", 512, False, False),     # MXFP4 bank kernels
    ("mxfp4", 512, False, True),      # MXFP4 bank on the block-scaled MFMA (MXFP8 rows)
])
def test_graph_replays_match_eager(name, T, backward, mx8):
    print(f"[graph replay] {name} T={T} backward={backward} mx8={mx8}", flush=True)
    p = make_inputs(CONFIGS[name], T=T)
    d = di.upload(p, DEV)
    graph_step, eager_step = Step(p, d, backward, mx8), Step(p, d, backward, mx8)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph_step.run()                     # warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_step.run()
    torch.cuda.synchronize()

    adt, H, E = p["adt"], p["H"], p["E"]
    for n, seed in enumerate((31, 32, 33)):
        rng = np.random.default_rng(seed)
        d["x"].copy_(di.tensor(to_storage(rng.normal(0, 1, (T, H)), adt), adt, DEV))
        d["logits"].copy_(torch.from_numpy(rng.normal(0, 1.5, (T, E)).astype(np.float32)))
        if backward:
            gout = di.tensor(to_storage(rng.normal(0, 1, (T, H)), adt), adt, DEV)
            graph_step.gout.copy_(gout)
            eager_step.gout.copy_(gout)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = graph_step.outputs()
        eager_step.run()                     # eager work between the replays
        torch.cuda.synchronize()
        want = eager_step.outputs()
        for key, ref in want.items():
            assert torch.equal(got[key], ref), f"{name} replay {n}: {key} differs from eager"
