"""First-order autograd over the library's forward and VJP calls.

Marshalling only, like :mod:`moeq`: every forward and every derivative is one of
the C-ABI calls, run on torch's current stream.  The contracts come from the
pages:

* ruda-tensor packed_experts.rs, ``PackedExpertAutodiffError``: packed scales,
  codebooks and biases stay frozen (``TrainableMetadata``), and the native input
  VJPs give first-order derivatives only (``HigherDerivativeUnsupported``);
  ``FrozenPackedExpertOps`` names the forward calls and their input VJPs.
* ruda-tensor frozen_awq.rs, ``FrozenAwqError::TrainableBase``: a frozen AWQ
  projection refuses trainable scales or bias; its input VJP applies the
  transpose of the same rounded coefficients and implies no weight gradients.
* ruda-tensor moe_exchange.rs, ``MoeDispatchOps``: the combine VJP (expert rows
  and FP32 weights), the COPY VJP of the dispatch, and the fixed-selection logit
  VJP of the routing weights.

Three functions are differentiable:

* :func:`moe_expert_ffn` -- moe_dispatch -> awq_grouped_swiglu ->
  awq_grouped_down -> moe_combine; gradients for ``x`` (combine VJP, chain input
  VJP, COPY VJP) and ``logits`` (combine weight VJP, logit VJP);
* :func:`frozen_awq` -- frozen_awq_forward with awq_input_backward;
* :func:`packed_expert` -- awq_expert_forward with awq_expert_input_backward.

A backward asked to build a graph (``create_graph=True``) raises
``HigherDerivativeUnsupported`` before any work; each backward is also wrapped
in torch's ``once_differentiable``.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import torch
from torch.autograd.function import once_differentiable

from . import moeq


class PackedExpertAutodiffError(RuntimeError):
    """packed_experts.rs PackedExpertAutodiffError (the non-native variants)."""
    TRAINABLE_METADATA = "TrainableMetadata"
    HIGHER_DERIVATIVE_UNSUPPORTED = "HigherDerivativeUnsupported"
    _TEXT = {TRAINABLE_METADATA: "packed expert quantization metadata and bias are frozen; "
                                 "a trainable scale or bias is not this operation",
             HIGHER_DERIVATIVE_UNSUPPORTED: "the packed expert input VJPs give first-order "
                                            "derivatives only"}

    def __init__(self, kind: str, detail: str = ""):
        super().__init__(f"{kind}: {self._TEXT[kind]}" + (f" ({detail})" if detail else ""))
        self.kind = kind


class FrozenAwqError(RuntimeError):
    """frozen_awq.rs FrozenAwqError::TrainableBase."""
    TRAINABLE_BASE = "TrainableBase"

    def __init__(self, detail: str = ""):
        super().__init__(f"{self.TRAINABLE_BASE}: a frozen AWQ projection takes no scales or "
                         "bias that require gradients" + (f" ({detail})" if detail else ""))
        self.kind = self.TRAINABLE_BASE


def _payload_tensors(name: str, w):
    if isinstance(w, moeq.AwqExperts):
        return [(f"{name}.qweight", w.qweight), (f"{name}.qzeros", w.qzeros),
                (f"{name}.scales", w.scales), (f"{name}.bias", w.bias)]
    if isinstance(w, moeq.Mxfp4Bank):
        return [(f"{name}.blocks", w.blocks), (f"{name}.scales", w.scales),
                (f"{name}.bias", w.bias)]
    raise TypeError(f"{name}: expected AwqExperts or Mxfp4Bank, got {type(w).__name__}")


def _trainable(payloads) -> list:
    return [nm for name, w in payloads if w is not None
            for nm, t in _payload_tensors(name, w) if t is not None and t.requires_grad]


def _first_order(backward):
    """Backward wrapper: refuse graph-building backward passes, then run the VJP
    under torch's once_differentiable (no graph is recorded through it)."""
    inner = once_differentiable(backward)

    @functools.wraps(backward)
    def wrapper(ctx, *grads):
        if torch.is_grad_enabled():     # create_graph=True: a higher derivative was asked for
            raise PackedExpertAutodiffError(
                PackedExpertAutodiffError.HIGHER_DERIVATIVE_UNSUPPORTED)
        return inner(ctx, *grads)
    return wrapper


# ------------------------------------------------------------------ routed FFN
@dataclasses.dataclass(frozen=True)
class _FfnSpec:
    top_k: int
    expert_bias: Optional[torch.Tensor]
    gate: object
    up: object
    down: object
    clamp: float
    alpha: float
    up_offset: float
    gate_one_sided: bool


class _MoeExpertFFN(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, logits, spec: _FfnSpec):
        d = moeq.moe_dispatch(x, logits, spec.expert_bias, spec.top_k)
        route = d["route"]
        h = moeq.awq_grouped_swiglu(route, d["values"], spec.gate, spec.up, spec.clamp,
                                    spec.alpha, spec.up_offset,
                                    gate_one_sided=spec.gate_one_sided)
        y = moeq.awq_grouped_down(route, h, spec.down)
        out = moeq.moe_combine(route, y, d["weights"])
        ctx.spec, ctx.route = spec, route
        ctx.save_for_backward(d["values"], y, d["weights"], d["selected"])
        return out

    @staticmethod
    @_first_order
    def backward(ctx, grad_out):
        spec, route = ctx.spec, ctx.route
        values, y, weights, selected = ctx.saved_tensors
        need_x, need_logits = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        grad_out = grad_out.contiguous()
        if grad_out.dtype != y.dtype:
            raise moeq.MoeqError(moeq.EDTYPE, "the output derivative keeps the activation dtype")
        gx = glogits = None
        gy, gw = moeq.moe_combine_backward(route, y, weights, grad_out, experts=need_x,
                                           want_weights=need_logits)
        if need_x:
            gv = moeq.awq_swiglu_input_backward(route, values, spec.gate, spec.up, spec.down,
                                                gy, spec.clamp, spec.alpha, spec.up_offset,
                                                gate_one_sided=spec.gate_one_sided)
            gx = moeq.moe_dispatch_backward(route, gv)
        if need_logits:
            glogits = moeq.moe_dispatch_weights_backward(route, selected, weights, gw)
        return gx, glogits, None


def moe_expert_ffn(x: torch.Tensor, logits: torch.Tensor, gate, up, down, top_k: int,
                   expert_bias: Optional[torch.Tensor] = None, clamp: float = 0.0,
                   alpha: float = 1.0, up_offset: float = 0.0,
                   gate_one_sided: bool = False) -> torch.Tensor:
    """Differentiable routed expert FFN: out [T, K] in x's dtype.

    x [T, K] (fp32 or bf16), logits [T, E] fp32, expert_bias [E] fp32 or None
    (a constant added to the logits); gate / up / down: AwqExperts (or an
    interleaved Mxfp4Bank as gate with up None, and a Mxfp4Bank as down, forward
    and logit derivative only).  Raises PackedExpertAutodiffError
    TrainableMetadata when any payload tensor requires a gradient."""
    bad = _trainable([("gate", gate), ("up", up), ("down", down)])
    if bad:
        raise PackedExpertAutodiffError(PackedExpertAutodiffError.TRAINABLE_METADATA,
                                        ", ".join(bad))
    if expert_bias is not None and expert_bias.requires_grad:
        raise PackedExpertAutodiffError(PackedExpertAutodiffError.TRAINABLE_METADATA,
                                        "the router's expert bias is a constant here")
    if x.requires_grad and isinstance(gate, moeq.Mxfp4Bank):
        raise moeq.MoeqError(moeq.EUNSUPPORTED, "the input VJP through MXFP4 banks is not "
                                                "implemented")
    spec = _FfnSpec(int(top_k), expert_bias, gate, up, down, float(clamp), float(alpha),
                    float(up_offset), bool(gate_one_sided))
    return _MoeExpertFFN.apply(x, logits, spec)


# ------------------------------------------------------------------ frozen projection
class _FrozenAwq(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, w):
        ctx.w = w
        return moeq.frozen_awq_forward(x2, w)

    @staticmethod
    @_first_order
    def backward(ctx, grad):
        return moeq.awq_input_backward(None, grad.contiguous(), ctx.w), None


def frozen_awq(x: torch.Tensor, w) -> torch.Tensor:
    """frozen_awq.rs frozen_awq_forward: y = x . W (+ b) with one packed matrix
    (a one-expert AwqExperts); the output keeps x's dtype and leading axes.  The
    input derivative is frozen_awq_input_backward (AWQ only).  Raises
    FrozenAwqError (TrainableBase) when scales or bias require gradients."""
    bad = _trainable([("w", w)])
    if bad:
        raise FrozenAwqError(", ".join(bad))
    if x.requires_grad and not isinstance(w, moeq.AwqExperts):
        raise moeq.MoeqError(moeq.EUNSUPPORTED, "the frozen input VJP is implemented for AWQ")
    lead = x.shape[:-1]
    y = _FrozenAwq.apply(x.reshape(-1, x.shape[-1]).contiguous(), w)
    return y.reshape(*lead, y.shape[-1])


# ------------------------------------------------------------------ rows in any order
class _PackedExpert(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, ids, w):
        ctx.w = w
        ctx.save_for_backward(ids)
        return moeq.awq_expert_forward(x2, ids, w)

    @staticmethod
    @_first_order
    def backward(ctx, grad):
        (ids,) = ctx.saved_tensors
        return moeq.awq_expert_input_backward(grad.contiguous(), ids, ctx.w), None, None


def packed_expert(x: torch.Tensor, global_ids: torch.Tensor, w) -> torch.Tensor:
    """packed_experts.rs packed_expert_forward: rows in any order, each with its
    global expert ID (int32/uint32 bits, one per row); output in the incoming
    order, x's dtype and leading axes.  Input derivative:
    packed_expert_input_backward (AWQ only).  Raises PackedExpertAutodiffError
    TrainableMetadata when scales or bias require gradients."""
    bad = _trainable([("w", w)])
    if bad:
        raise PackedExpertAutodiffError(PackedExpertAutodiffError.TRAINABLE_METADATA,
                                        ", ".join(bad))
    if x.requires_grad and not isinstance(w, moeq.AwqExperts):
        raise moeq.MoeqError(moeq.EUNSUPPORTED, "the packed input VJP is implemented for AWQ")
    lead = x.shape[:-1]
    ids = global_ids.reshape(-1).contiguous()
    y = _PackedExpert.apply(x.reshape(-1, x.shape[-1]).contiguous(), ids, w)
    return y.reshape(*lead, y.shape[-1])
