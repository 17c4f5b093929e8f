"""Host-side checks of the autograd layer and of the binding's payload validation.

No GPU and no library call: every rejection here happens before anything is
enqueued.  Contracts: ruda-tensor packed_experts.rs PackedExpertAutodiffError
(TrainableMetadata, HigherDerivativeUnsupported); frozen_awq.rs FrozenAwqError
(TrainableBase); the AWQ payload shapes of packed_experts.rs AwqExpertPayload
and the MXFP4 bank shapes of libmir-metal native.rs validate.
"""
import pytest
import torch

from quantized_moe_expert_router_amd import autograd as ag
from quantized_moe_expert_router_amd import moeq


def awq_payload(E=2, K=64, N=16, g=32, sdt=torch.bfloat16, bias=True):
    return moeq.AwqExperts(torch.zeros(E, K, N // 8, dtype=torch.int32),
                           torch.zeros(E, K // g, N // 8, dtype=torch.int32),
                           torch.ones(E, K // g, N, dtype=sdt), g,
                           torch.zeros(E, N, dtype=sdt) if bias else None)


def bank(E=2, R=32, C=64, inter=True):
    return moeq.Mxfp4Bank(torch.zeros(E, R, C // 32, 16, dtype=torch.uint8),
                          torch.full((E, R, C // 32), 127, dtype=torch.uint8),
                          torch.zeros(E, R, dtype=torch.bfloat16), inter)


@pytest.mark.parametrize("which", ["gate", "up", "down"])
@pytest.mark.parametrize("field", ["scales", "bias"])
def test_ffn_rejects_trainable_metadata(which, field):
    w = {nm: awq_payload() for nm in ("gate", "up", "down")}
    getattr(w[which], field).requires_grad_(True)
    x = torch.zeros(4, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ag.PackedExpertAutodiffError) as ei:
        ag.moe_expert_ffn(x, torch.zeros(4, 2), w["gate"], w["up"], w["down"], 1)
    assert ei.value.kind == "TrainableMetadata"
    assert f"{which}.{field}" in str(ei.value)


def test_ffn_rejects_trainable_bank_bias():
    gu, dn = bank(R=32), bank(R=64, C=32, inter=False)
    gu.bias.requires_grad_(True)
    with pytest.raises(ag.PackedExpertAutodiffError) as ei:
        ag.moe_expert_ffn(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 2), gu,
                          None, dn, 1)
    assert ei.value.kind == "TrainableMetadata"


def test_ffn_rejects_trainable_router_bias():
    w = awq_payload()
    with pytest.raises(ag.PackedExpertAutodiffError):
        ag.moe_expert_ffn(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 2), w, w, w,
                          1, expert_bias=torch.zeros(2, requires_grad=True))


def test_ffn_bank_input_vjp_unsupported():
    gu, dn = bank(R=32), bank(R=64, C=32, inter=False)
    x = torch.zeros(4, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(moeq.MoeqError) as ei:
        ag.moe_expert_ffn(x, torch.zeros(4, 2), gu, None, dn, 1)
    assert ei.value.status == moeq.EUNSUPPORTED


@pytest.mark.parametrize("field", ["scales", "bias"])
def test_frozen_awq_rejects_trainable_base(field):
    w = awq_payload(E=1)
    getattr(w, field).requires_grad_(True)
    with pytest.raises(ag.FrozenAwqError) as ei:
        ag.frozen_awq(torch.zeros(3, 64, dtype=torch.bfloat16), w)
    assert ei.value.kind == "TrainableBase"


def test_packed_expert_rejects_trainable_metadata():
    w = awq_payload()
    w.scales.requires_grad_(True)
    with pytest.raises(ag.PackedExpertAutodiffError):
        ag.packed_expert(torch.zeros(3, 64, dtype=torch.bfloat16),
                         torch.zeros(3, dtype=torch.int32), w)


class _Twice(torch.autograd.Function):
    """A stand-in with a first-order backward, to exercise the wrapper on the CPU."""

    @staticmethod
    def forward(ctx, x):
        return x * 2

    @staticmethod
    @ag._first_order
    def backward(ctx, g):
        return g * 2


def test_first_order_only():
    x = torch.ones(3, requires_grad=True)
    (gx,) = torch.autograd.grad(_Twice.apply(x).sum(), x)
    assert torch.equal(gx, torch.full((3,), 2.0))
    with pytest.raises(ag.PackedExpertAutodiffError) as ei:
        torch.autograd.grad(_Twice.apply(x).sum(), x, create_graph=True)
    assert ei.value.kind == "HigherDerivativeUnsupported"
    # the derivative computed without a graph cannot be differentiated again
    assert not gx.requires_grad


@pytest.mark.parametrize("case,status", [
    ("bias_dtype", moeq.EDTYPE), ("bias_shape", moeq.ESHAPE), ("scales_shape", moeq.ESHAPE),
    ("qzeros_shape", moeq.ESHAPE), ("qweight_dtype", moeq.EDTYPE), ("scales_dtype", moeq.EDTYPE),
    ("group", moeq.ESHAPE), ("rank", moeq.ESHAPE)])
def test_awq_payload_validation(case, status):
    w = awq_payload(sdt=torch.float32)
    if case == "bias_dtype":      # a bf16 bias beside fp32 scales would be read as fp32
        w.bias = w.bias.to(torch.bfloat16)
    elif case == "bias_shape":
        w.bias = torch.zeros(2, 8, dtype=torch.float32)
    elif case == "scales_shape":
        w.scales = torch.ones(2, 2, 8, dtype=torch.float32)
    elif case == "qzeros_shape":
        w.qzeros = torch.zeros(2, 1, 2, dtype=torch.int32)
    elif case == "qweight_dtype":
        w.qweight = w.qweight.to(torch.int64)
    elif case == "scales_dtype":
        w.scales = w.scales.to(torch.float64)
    elif case == "group":
        w.group_size = 48
    elif case == "rank":
        w.qweight = w.qweight[0]
    with pytest.raises(moeq.MoeqError) as ei:
        w.c()
    assert ei.value.status == status
    awq_payload(sdt=torch.float32).c()          # the unmodified payload passes


@pytest.mark.parametrize("case,status", [
    ("bias_dtype", moeq.EDTYPE), ("bias_shape", moeq.ESHAPE), ("scales_shape", moeq.ESHAPE),
    ("blocks_dtype", moeq.EDTYPE), ("no_bias", moeq.EDTYPE)])
def test_bank_validation(case, status):
    b = bank()
    if case == "bias_dtype":
        b.bias = b.bias.float()
    elif case == "bias_shape":
        b.bias = torch.zeros(2, 16, dtype=torch.bfloat16)
    elif case == "scales_shape":
        b.scales = torch.zeros(2, 32, 1, dtype=torch.uint8)
    elif case == "blocks_dtype":
        b.blocks = b.blocks.to(torch.int8)
    elif case == "no_bias":
        b.bias = None
    with pytest.raises(moeq.MoeqError) as ei:
        b.c()
    assert ei.value.status == status
    bank().c()
