"""GPU parity of the rows-in-any-order calls against the CPU oracle, through the C-ABI.

packed_experts.rs packed_expert_forward / packed_expert_input_backward
(awq_expert_forward / awq_expert_input_backward: local sort by global ID, the
grouped kernels, inverse permutation) and frozen_awq.rs frozen_awq_forward (one
cube over all rows).  Bars: the projection tolerance, max relative row error
1e-4 (fp32 activations) / 2e-2 (bf16); bit-exact where every product and sum is
exact (power-of-two scales, small-integer activations), which pins the row
permutation and its inverse; bit-exact against the routed grouped kernels on the
same rows (the restore is a pure copy).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, TOL, f64, row_rel_err
from quantized_moe_expert_router_amd import device_inputs as di
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd.synth import awq_cube, to_storage

pytestmark = pytest.mark.gpu


def cube(seed, E, K, N, g, sdt, bias=False, exact=False):
    rng = np.random.default_rng(seed)
    qw, qz, s, b = awq_cube(rng, E, K, N, g, sdt, 0.002, 0.01, bias)
    if exact:
        s = to_storage((2.0 ** -rng.integers(6, 9, size=s.shape)).astype(np.float64), sdt)
    dev = moeq.AwqExperts(di.tensor(qw, "i32", DEV), di.tensor(qz, "i32", DEV),
                          di.tensor(s, sdt, DEV), g, None if b is None else di.tensor(b, sdt, DEV))
    return (qw, qz, s, b), dev


def ids_tensor(ids):
    return torch.from_numpy(np.ascontiguousarray(ids, np.uint32).view(np.int32)).to(DEV)


@pytest.mark.parametrize("rows,E,K,N,g,sdt,adt,start,bias", [
    (37, 16, 256, 512, 128, "bf16", "bf16", 0, False),    # few rows per expert: stream kernel
    (900, 8, 512, 256, 64, "f16", "bf16", 0, True),       # many rows: register-decoded kernel
    (700, 6, 384, 256, 128, "f32", "bf16", 24, True),     # fp32 scales, a resident range at 24
    (50, 4, 128, 64, 32, "f16", "f32", 8, True),          # fp32 activations: generic kernel
    (1, 3, 128, 128, 64, "bf16", "bf16", 0, False),       # one row
])
def test_expert_forward_any_order(rows, E, K, N, g, sdt, adt, start, bias):
    print(f"[awq_expert_forward] rows={rows} E={E} K={K} N={N} g={g} {sdt}/{adt} start={start}",
          flush=True)
    host, dev = cube(71, E, K, N, g, sdt, bias)
    dev.expert_start = start
    rng = np.random.default_rng(72)
    x = to_storage(rng.normal(0, 1, (rows, K)), adt)
    local = rng.integers(0, E, size=rows)
    local[: rows // 3] = 1                               # one heavier expert, order mixed
    rng.shuffle(local)
    y = moeq.awq_expert_forward(di.tensor(x, adt, DEV), ids_tensor(local + start), dev)
    torch.cuda.synchronize()
    ref = oracle.awq_project(x, adt, local.astype(np.uint32), host[0], host[1], host[2], sdt, g,
                             bias=host[3])
    assert row_rel_err(f64(di.to_host(y, adt), adt), f64(ref, adt)) <= TOL[adt]
    # the input VJP in the incoming order (AWQ)
    grad = to_storage(rng.normal(0, 1, (rows, N)), adt)
    gi = moeq.awq_expert_input_backward(di.tensor(grad, adt, DEV), ids_tensor(local + start), dev)
    torch.cuda.synchronize()
    refg = oracle.awq_input_backward(grad, adt, local.astype(np.uint32), host[0], host[1],
                                     host[2], sdt, g)
    assert row_rel_err(f64(di.to_host(gi, adt), adt), f64(refg, adt)) <= TOL[adt]


@pytest.mark.parametrize("rows,E", [(60, 8), (800, 8)])
def test_expert_forward_exact_permutation(rows, E):
    """Exact arithmetic: the result must equal the oracle bit for bit, so any row
    placed at the wrong incoming position fails."""
    print(f"[awq_expert_forward exact] rows={rows} E={E}", flush=True)
    host, dev = cube(73, E, 256, 256, 64, "bf16", exact=True)
    rng = np.random.default_rng(74)
    x = to_storage(rng.integers(-2, 3, size=(rows, 256)).astype(np.float64), "bf16")
    local = rng.integers(0, E, size=rows).astype(np.uint32)
    y = moeq.awq_expert_forward(di.tensor(x, "bf16", DEV), ids_tensor(local), dev)
    torch.cuda.synchronize()
    ref = oracle.awq_project(x, "bf16", local, host[0], host[1], host[2], "bf16", 64)
    np.testing.assert_array_equal(di.to_host(y, "bf16"), ref)


def test_expert_forward_matches_grouped_kernels():
    """Against the routed path: rows dispatched with top_k 1 and projected with
    awq_grouped_down, then returned through the combine with weight 1."""
    print("[awq_expert_forward vs grouped]", flush=True)
    E, K, N, T = 32, 512, 256, 300
    host, dev = cube(75, E, K, N, 128, "bf16")
    rng = np.random.default_rng(76)
    x = to_storage(rng.normal(0, 1, (T, K)), "bf16")
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    disp = moeq.moe_dispatch(di.tensor(x, "bf16", DEV), torch.from_numpy(logits).to(DEV), None, 1)
    ys = moeq.awq_grouped_down(disp["route"], disp["values"], dev)
    ids = disp["selected"].view(-1).contiguous()
    y = moeq.awq_expert_forward(di.tensor(x, "bf16", DEV), ids, dev)
    torch.cuda.synchronize()
    pos = disp["route"].slot_pos.view(-1).long()
    assert torch.equal(y, ys[pos])


def test_expert_forward_mxfp4_bank():
    print("[awq_expert_forward mxfp4]", flush=True)
    rng = np.random.default_rng(77)
    E, K, R, rows = 6, 256, 128, 90
    blocks = rng.integers(0, 256, size=(E, R, K // 32, 16), dtype=np.uint8)
    scales = rng.integers(119, 126, size=(E, R, K // 32), dtype=np.uint8)
    bias = to_storage(rng.normal(0, 0.01, size=(E, R)), "bf16")
    bank = moeq.Mxfp4Bank(di.tensor(blocks, "u8", DEV), di.tensor(scales, "u8", DEV),
                          di.tensor(bias, "bf16", DEV), False)
    x = to_storage(rng.normal(0, 1, (rows, K)), "bf16")
    local = rng.integers(0, E, size=rows).astype(np.uint32)
    y = moeq.awq_expert_forward(di.tensor(x, "bf16", DEV), ids_tensor(local), bank)
    torch.cuda.synchronize()
    ref = oracle.mxfp4_project(x, "bf16", local, blocks, scales, bias)
    assert row_rel_err(f64(di.to_host(y, "bf16"), "bf16"), f64(ref, "bf16")) <= TOL["bf16"]


def test_expert_forward_rejects_foreign_ids():
    print("[awq_expert_forward ERANGE]", flush=True)
    host, dev = cube(78, 4, 128, 64, 64, "bf16")
    dev.expert_start = 8
    x = torch.zeros(5, 128, dtype=torch.bfloat16, device=DEV)
    y = torch.full((5, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    for bad in ([8, 9, 12, 10, 11], [8, 9, 7, 10, 11]):
        with pytest.raises(moeq.MoeqError) as ei:
            moeq.awq_expert_forward(x, ids_tensor(bad), dev, y=y)
        assert ei.value.status == moeq.ERANGE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)                          # outputs untouched
    assert moeq.awq_expert_forward(x[:0], ids_tensor([]), dev).shape == (0, 64)


@pytest.mark.parametrize("rows,K,N,g,sdt,adt", [
    (5, 512, 256, 128, "bf16", "bf16"),     # stream kernel
    (700, 512, 384, 64, "f16", "bf16"),     # register-decoded kernel, several m-tiles
    (300, 256, 256, 128, "f32", "bf16"),    # fp32 scales
    (33, 128, 64, 32, "f16", "f32"),        # fp32 activations
])
def test_frozen_awq_forward(rows, K, N, g, sdt, adt):
    print(f"[frozen_awq_forward] rows={rows} K={K} N={N} g={g} {sdt}/{adt}", flush=True)
    host, dev = cube(79, 1, K, N, g, sdt, bias=True)
    x = to_storage(np.random.default_rng(80).normal(0, 1, (rows, K)), adt)
    y = moeq.frozen_awq_forward(di.tensor(x, adt, DEV), dev)
    torch.cuda.synchronize()
    ref = oracle.awq_project(x, adt, None, host[0], host[1], host[2], sdt, g, bias=host[3])
    assert row_rel_err(f64(di.to_host(y, adt), adt), f64(ref, adt)) <= TOL[adt]
