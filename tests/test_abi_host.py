"""The C-ABI library loads, exports every symbol of include/moeq.h, and rejects
invalid arguments on the host (no device work is enqueued on these paths).

Validation rules follow the pages: N % 8 and complete groups (packed_experts.rs
AwqExpertOptions), frozen metadata / no dense fallback (frozen_awq.rs
FrozenAwqError), the interleaved-bank and companion checks of native.rs
(native_layout, companions, validate, and its requires_typed_interleaved_expert_bank
test), and the expert-prefix ranges of moe_exchange.rs moe_dispatch_counts.
"""
import ctypes as C
import os
import re
import subprocess

import pytest

from quantized_moe_expert_router_amd import moeq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000          # never dereferenced: every call below fails validation first


def header_functions():
    text = open(os.path.join(ROOT, "include", "moeq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def L():
    return moeq.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert set(names) == set(moeq.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", moeq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings(L):
    for st in range(0, -8, -1):
        assert L.moeq_status_string(st).decode()
    assert b"fallback" in L.moeq_status_string(moeq.EUNSUPPORTED)


def bind(L, T, E, k, ptr=FAKE, nbytes=None):
    r = moeq.Route()
    if nbytes is None:
        nbytes = L.moeq_route_workspace_bytes(T, E, k)
    return L.moeq_route_bind(C.byref(r), C.c_void_p(ptr), nbytes, T, E, k), r


def test_route_layout(L):
    assert L.moeq_route_workspace_bytes(64, 128, 8) > 0
    for bad in [(-1, 8, 2), (4, 0, 1), (4, 8, 0), (4, 8, 9)]:
        assert L.moeq_route_workspace_bytes(*bad) == 0
    st, r = bind(L, 300, 128, 8)
    assert st == moeq.OK and r.T == 300 and r.E == 128 and r.top_k == 8
    n = L.moeq_route_workspace_bytes(300, 128, 8)
    spans = sorted([(r.expert_offsets, 4 * 129), (r.row_src, 4 * 2400), (r.slot_pos, 4 * 2400),
                    (r.block_base, 4 * 2 * 128), (r.tile_offsets, 4 * 129),
                    (r.tile_expert, 4 * (19 + 128))])
    for (a, la), (b, _) in zip(spans, spans[1:]):
        assert a + la <= b                           # disjoint
    assert spans[0][0] >= FAKE and spans[-1][0] + spans[-1][1] <= FAKE + n
    assert all(p % 256 == 0 for p, _ in spans)


def test_route_bind_errors(L):
    r = moeq.Route()
    assert L.moeq_route_bind(C.byref(r), None, 1 << 20, 4, 8, 2) == moeq.EINVAL
    assert bind(L, 4, 8, 2, ptr=FAKE + 4)[0] == moeq.EWORKSPACE
    assert bind(L, 4, 8, 2, nbytes=16)[0] == moeq.EWORKSPACE
    assert b"workspace" in L.moeq_last_error()
    assert bind(L, 4, 8, 9)[0] == moeq.EINVAL


def dispatch(L, route, T=4, E=8, k=2, K=16, act=moeq.BF16, ptr=FAKE, ldt=moeq.F32):
    p = C.c_void_p(ptr)
    return L.moe_dispatch(p, act, T, K, p, ldt, E, None, k, p, p, p, p, C.byref(route), None)


def test_dispatch_validation(L):
    assert dispatch(L, moeq.Route()) == moeq.EINVAL            # unbound route
    st, r = bind(L, 4, 8, 2)
    assert dispatch(L, r, T=5) == moeq.ESHAPE
    assert dispatch(L, r, k=3) == moeq.ESHAPE
    assert dispatch(L, r, act=7) == moeq.EDTYPE
    assert dispatch(L, r, ldt=moeq.F16) == moeq.EDTYPE          # logits: fp32 or bf16
    assert b"logits" in L.moeq_last_error()
    assert dispatch(L, r, ldt=9) == moeq.EDTYPE
    assert dispatch(L, r, K=0) == moeq.EINVAL
    assert dispatch(L, r, ptr=0) == moeq.EINVAL                 # NULL tensors
    st, r = bind(L, 4, 4096, 2)
    assert dispatch(L, r, E=4096) == moeq.EUNSUPPORTED
    st, r = bind(L, 4, 64, 33)
    assert dispatch(L, r, E=64, k=33) == moeq.EUNSUPPORTED
    st, r = bind(L, 0, 8, 2)
    assert dispatch(L, r, T=0) == moeq.OK                        # T = 0 is a no-op


def counts(L, r, prefix):
    pre = (C.c_int64 * len(prefix))(*prefix)
    out = (C.c_int64 * max(len(prefix) - 1, 1))()
    st = L.moe_dispatch_counts(C.byref(r), C.cast(pre, C.c_void_p), len(prefix) - 1,
                               C.cast(out, C.c_void_p), None)
    return st, list(out)[:max(len(prefix) - 1, 0)]


def test_counts_validation(L):
    _, r = bind(L, 4, 8, 2)
    assert counts(L, r, [0, 9])[0] == moeq.ERANGE
    assert counts(L, r, [0, 5, 3])[0] == moeq.ERANGE
    assert counts(L, r, [-1, 3])[0] == moeq.ERANGE
    assert counts(L, r, [3])[0] == moeq.OK                       # R = 0: nothing to count
    _, r0 = bind(L, 0, 8, 2)
    assert counts(L, r0, [0, 3, 8]) == (moeq.OK, [0, 0])          # no tokens: no copy


def awq(E=8, K=64, N=32, g=32, sdt=moeq.BF16, qz=FAKE, bias=None, start=0):
    return moeq.Experts(moeq.FMT_AWQ, E, start, K, N, g, FAKE, qz, FAKE, sdt, bias, 0)


def bank(E=8, K=64, R=64, inter=1, bias=FAKE):
    return moeq.Experts(moeq.FMT_MXFP4_BANK, E, 0, K, R, 32, FAKE, None, FAKE, moeq.BF16, bias,
                        inter)


def swiglu(L, r, gate, up, act=moeq.BF16, fn=(0.0, 1.0, 0.0)):
    return L.awq_grouped_swiglu(C.byref(r), C.c_void_p(FAKE), act, C.byref(gate),
                                None if up is None else C.byref(up), moeq.SwiGLU(*fn),
                                C.c_void_p(FAKE), None)


def test_projection_validation(L):
    _, r = bind(L, 0, 8, 2)       # A = 0: a valid call enqueues nothing and returns OK
    assert swiglu(L, r, awq(), awq()) == moeq.OK
    assert swiglu(L, r, awq(N=36), awq(N=36)) == moeq.ESHAPE          # N % 8
    assert swiglu(L, r, awq(K=48), awq(K=48)) == moeq.ESHAPE          # K % g
    assert swiglu(L, r, awq(g=16, K=64), awq(g=16, K=64)) == moeq.EUNSUPPORTED
    assert swiglu(L, r, awq(E=4), awq(E=4)) == moeq.ERANGE            # must cover [0, E)
    assert swiglu(L, r, awq(start=1, E=8), awq(start=1)) == moeq.ERANGE
    assert swiglu(L, r, awq(), awq(N=64)) == moeq.ESHAPE              # gate/up mismatch
    assert swiglu(L, r, awq(), awq(sdt=moeq.F16)) == moeq.EDTYPE
    assert swiglu(L, r, awq(sdt=9), awq(sdt=9)) == moeq.EDTYPE
    assert swiglu(L, r, awq(qz=None), awq()) == moeq.EINVAL
    assert swiglu(L, r, awq(), awq(bias=FAKE)) == moeq.EINVAL
    assert swiglu(L, r, awq(), None) == moeq.EINVAL
    assert swiglu(L, r, awq(), awq(), act=moeq.F16) == moeq.OK   # fp16 rows: VALU kernels
    assert swiglu(L, r, awq(), awq(), act=5) == moeq.EDTYPE
    assert swiglu(L, r, awq(), awq(), fn=(-1.0, 1.0, 0.0)) == moeq.EINVAL
    assert swiglu(L, r, awq(), awq(), fn=(7.0, 1.702, 1.0, 1)) == moeq.OK   # one-sided gate
    assert swiglu(L, r, awq(), awq(), fn=(7.0, 1.702, 1.0, 2)) == moeq.EINVAL
    # MXFP4 banks (native.rs): the gate/up role requires an interleaved bank with bias
    assert swiglu(L, r, bank(), None) == moeq.OK
    assert swiglu(L, r, bank(inter=0), None) == moeq.ESHAPE
    assert b"interleaved" in L.moeq_last_error()
    assert swiglu(L, r, bank(bias=None), None) == moeq.EINVAL
    assert swiglu(L, r, bank(K=48), None) == moeq.ESHAPE
    assert swiglu(L, r, bank(R=63), None) == moeq.ESHAPE
    assert swiglu(L, r, bank(), bank()) == moeq.EINVAL


def test_down_and_backward_validation(L):
    _, r = bind(L, 0, 8, 2)
    d = lambda w, act=moeq.BF16: L.awq_grouped_down(C.byref(r), C.c_void_p(FAKE), act,
                                                    C.byref(w), C.c_void_p(FAKE), None)
    assert d(awq()) == moeq.OK
    assert d(bank(inter=0)) == moeq.OK
    assert d(bank(inter=1)) == moeq.ESHAPE          # matrix-bank layout differs from role
    assert d(awq(N=12)) == moeq.ESHAPE
    b = lambda route, rows, w, gdt=moeq.F32: L.awq_input_backward(
        route, C.c_void_p(FAKE), gdt, rows, C.byref(w), C.c_void_p(FAKE), None)
    assert b(C.byref(r), 0, awq()) == moeq.OK
    assert b(C.byref(r), 3, awq()) == moeq.ESHAPE    # rows must equal the routed rows
    assert b(None, 0, awq(E=1)) == moeq.OK           # single frozen projection
    assert b(None, 4, awq(E=2)) == moeq.ERANGE
    assert b(None, 4, bank(E=1, inter=0)) == moeq.EUNSUPPORTED
    assert b(None, 0, awq(E=1), gdt=moeq.F16) == moeq.OK
    assert b(None, 4, awq(E=1), gdt=7) == moeq.EDTYPE
    assert b(None, -1, awq(E=1)) == moeq.EINVAL


def test_combine_validation(L):
    _, r = bind(L, 4, 8, 2)
    c = lambda K=16, act=moeq.BF16, ptr=FAKE: L.moe_combine(C.byref(r), C.c_void_p(ptr), act, K,
                                                           C.c_void_p(ptr), C.c_void_p(ptr), None)
    assert c(K=0) == moeq.EINVAL
    assert c(act=3) == moeq.EDTYPE
    assert c(ptr=0) == moeq.EINVAL


def test_size_overflow_is_rejected(L):
    _, r = bind(L, 0, 8, 2)
    for E, K, N in [(8, 1 << 30, 1 << 30), ((1 << 30), (1 << 30), 1 << 30)]:
        big = awq(E=E, K=K, N=N, g=1 << 30)
        assert swiglu(L, r, big, big) in (moeq.ESHAPE, moeq.ERANGE)
        assert b"overflow" in L.moeq_last_error() or b"cover" in L.moeq_last_error()
    _, r = bind(L, 0, 1 << 30, 2)
    big = awq(E=1 << 30, K=1 << 30, N=1 << 30, g=1 << 30)
    assert swiglu(L, r, big, big) == moeq.ESHAPE


def test_backward_path_validation(L):
    """moe_exchange.rs MoeDispatchOps backward calls and packed_experts.rs
    packed_swiglu_input_backward: every case below fails validation or is a no-op."""
    P = C.c_void_p(FAKE)
    _, r = bind(L, 4, 8, 2)
    _, r0 = bind(L, 0, 8, 2)
    _, r33 = bind(L, 4, 64, 33)
    cb = lambda route, K=16, act=moeq.BF16, grad=P, gy=P, gw=P: L.moe_combine_backward(
        C.byref(route), P, act, K, P, grad, gy, gw, None)
    assert cb(r, K=0) == moeq.EINVAL
    assert cb(r, act=3) == moeq.EDTYPE
    assert cb(r, grad=None) == moeq.EINVAL
    assert cb(r, gy=None, gw=None) == moeq.OK          # nothing requested: nothing formed
    assert cb(r0) == moeq.OK
    assert cb(r33) == moeq.EUNSUPPORTED
    assert L.moe_combine_backward(C.byref(moeq.Route()), P, moeq.BF16, 16, P, P, P, P,
                                  None) == moeq.EINVAL
    db = lambda route, K=16, act=moeq.BF16, ptr=P: L.moe_dispatch_backward(
        C.byref(route), ptr, act, K, ptr, None)
    assert db(r, K=0) == moeq.EINVAL
    assert db(r, act=9) == moeq.EDTYPE
    assert db(r, ptr=None) == moeq.EINVAL
    assert db(r0) == moeq.OK
    assert db(r33) == moeq.EUNSUPPORTED
    wb = lambda route, ptr=P: L.moe_dispatch_weights_backward(C.byref(route), ptr, ptr, ptr, ptr,
                                                              None)
    assert wb(r, ptr=None) == moeq.EINVAL
    assert wb(r0) == moeq.OK
    assert wb(r33) == moeq.EUNSUPPORTED
    ws = L.awq_swiglu_input_backward_workspace_bytes
    assert ws(8, 32, moeq.BF16) >= 2 * 8 * 32 * 2 and ws(8, 32, moeq.BF16) % 256 == 0
    assert ws(0, 32, moeq.F32) > 0
    assert ws(-1, 32, moeq.BF16) == 0 and ws(8, 0, moeq.BF16) == 0 and ws(8, 32, 7) == 0
    need = ws(8, 32, moeq.BF16)

    def sib(route, gate=None, up=None, down=None, act=moeq.BF16, fn=(0.0, 1.0, 0.0),
            wsp=FAKE, nbytes=need):
        gate = gate or awq(K=64, N=32)
        up = up or awq(K=64, N=32)
        down = down or awq(K=32, N=64)
        return L.awq_swiglu_input_backward(C.byref(route), P, act, C.byref(gate), C.byref(up),
                                           C.byref(down), moeq.SwiGLU(*fn), P, P,
                                           C.c_void_p(wsp) if wsp else None, nbytes, None)
    assert sib(r0) == moeq.OK                           # no rows: nothing enqueued
    assert sib(r, wsp=0) == moeq.EINVAL
    assert sib(r, wsp=FAKE + 16) == moeq.EWORKSPACE
    assert sib(r, nbytes=need - 1) == moeq.EWORKSPACE
    assert sib(r, down=awq(K=32, N=48)) == moeq.ESHAPE  # down must map I back to K
    assert sib(r, up=awq(K=64, N=40)) == moeq.ESHAPE
    assert sib(r, up=awq(K=64, N=32, sdt=moeq.F16)) == moeq.EDTYPE
    assert sib(r, gate=awq(K=64, N=32, bias=FAKE)) == moeq.EINVAL
    assert sib(r, down=bank(K=32, R=64, inter=0)) == moeq.EUNSUPPORTED
    assert sib(r0, act=moeq.F16) == moeq.OK              # fp16 rows: VALU kernels
    assert sib(r, act=6) == moeq.EDTYPE
    assert sib(r, fn=(-2.0, 1.0, 0.0)) == moeq.EINVAL
    assert sib(r, down=awq(E=4, K=32, N=64)) == moeq.ERANGE


def test_unsorted_and_single_projection_validation(L):
    """packed_experts.rs packed_expert_forward / packed_expert_input_backward and
    frozen_awq.rs frozen_awq_forward: every case fails validation before any device
    work, or is a no-op (rows = 0)."""
    P = C.c_void_p(FAKE)
    ws = L.awq_expert_workspace_bytes
    assert ws(100, 8, 64, 32, moeq.BF16) > 0 and ws(100, 8, 64, 32, moeq.BF16) % 256 == 0
    assert ws(0, 8, 64, 32, moeq.BF16) > 0
    assert ws(-1, 8, 64, 32, moeq.BF16) == 0 and ws(4, 0, 64, 32, moeq.BF16) == 0
    assert ws(4, 8, 0, 32, moeq.BF16) == 0 and ws(4, 8, 64, 32, 5) == 0
    need = ws(100, 8, 64, 32, moeq.BF16)

    def fwd(rows=100, w=None, act=moeq.BF16, x=FAKE, ids=FAKE, y=FAKE, wsp=FAKE, nbytes=need):
        w = w or awq(E=8, K=64, N=32)
        v = lambda a: C.c_void_p(a) if a else None
        return L.awq_expert_forward(v(x), act, rows, v(ids), C.byref(w), v(y), v(wsp), nbytes,
                                    None)
    assert fwd(rows=0) == moeq.OK
    assert fwd(rows=-1) == moeq.EINVAL
    assert fwd(act=4) == moeq.EDTYPE
    assert fwd(rows=0, act=moeq.F16) == moeq.OK        # fp16 rows pass the dtype check
    assert fwd(act=moeq.F16, y=0) == moeq.EINVAL
    assert fwd(w=awq(E=8, K=64, N=36)) == moeq.ESHAPE
    assert fwd(w=awq(E=4096, K=64, N=32)) == moeq.EUNSUPPORTED
    assert fwd(y=0) == moeq.EINVAL
    assert fwd(wsp=0) == moeq.EINVAL
    assert fwd(wsp=FAKE + 64) == moeq.EWORKSPACE
    assert fwd(nbytes=need - 1) == moeq.EWORKSPACE
    assert fwd(x=0) == moeq.EINVAL
    assert fwd(ids=0) == moeq.EINVAL
    assert fwd(w=bank(E=8, K=64, R=32, inter=1)) == moeq.ESHAPE   # a plain role takes a plain bank

    def bwd(rows=100, w=None, gdt=moeq.BF16, wsp=FAKE, nbytes=need):
        w = w or awq(E=8, K=64, N=32)
        return L.awq_expert_input_backward(P, gdt, rows, P, C.byref(w), P,
                                           C.c_void_p(wsp) if wsp else None, nbytes, None)
    assert bwd(rows=0) == moeq.OK
    assert bwd(rows=0, gdt=moeq.F16) == moeq.OK
    assert bwd(gdt=moeq.F16, wsp=0) == moeq.EINVAL
    assert bwd(w=bank(E=8, K=64, R=32, inter=0)) == moeq.EUNSUPPORTED
    assert bwd(wsp=0) == moeq.EINVAL
    assert bwd(nbytes=16) == moeq.EWORKSPACE

    fw = L.frozen_awq_workspace_bytes
    assert fw(0) > 0 and fw(1000) >= fw(10) and fw(-1) == 0
    need1 = fw(300)

    def single(rows=300, w=None, act=moeq.BF16, wsp=FAKE, nbytes=need1, x=FAKE):
        w = w or awq(E=1, K=64, N=32)
        return L.frozen_awq_forward(C.c_void_p(x) if x else None, act, rows, C.byref(w), P,
                                    C.c_void_p(wsp) if wsp else None, nbytes, None)
    assert single(rows=0) == moeq.OK
    assert single(w=awq(E=2, K=64, N=32)) == moeq.ERANGE
    assert single(rows=0, act=moeq.F16) == moeq.OK
    assert single(act=moeq.F16, x=0) == moeq.EINVAL
    assert single(x=0) == moeq.EINVAL
    assert single(wsp=0) == moeq.EINVAL
    assert single(nbytes=need1 - 1) == moeq.EWORKSPACE
    assert single(wsp=FAKE + 8) == moeq.EWORKSPACE


def test_mx8_validation(L):
    """The block-scaled MFMA path takes MXFP4 banks and bf16 rows only."""
    P = C.c_void_p(FAKE)
    assert L.mx8_workspace_bytes(100, 2880) >= 100 * 2880 + 100 * 90
    assert L.mx8_workspace_bytes(100, 48) == 0 and L.mx8_workspace_bytes(-1, 64) == 0
    assert L.mx8_quantize(P, moeq.F32, 4, 64, P, P, None) == moeq.EUNSUPPORTED
    assert L.mx8_quantize(P, moeq.BF16, 4, 48, P, P, None) == moeq.ESHAPE
    assert L.mx8_quantize(P, moeq.BF16, 0, 64, P, P, None) == moeq.OK
    assert L.mx8_quantize(None, moeq.BF16, 4, 64, P, P, None) == moeq.EINVAL
    _, r = bind(L, 4, 8, 2)
    _, r0 = bind(L, 0, 8, 2)
    need = L.mx8_workspace_bytes(8, 64)
    fn = moeq.SwiGLU(7.0, 1.0, 0.0, 0)
    sw = lambda route, w, act=moeq.BF16, wsp=FAKE, nbytes=need: L.mx8_grouped_swiglu(
        C.byref(route), P, act, C.byref(w), fn, P, C.c_void_p(wsp) if wsp else None, nbytes, None)
    assert sw(r0, bank(K=64, R=128)) == moeq.OK
    assert sw(r, awq()) == moeq.EUNSUPPORTED
    assert sw(r, bank(K=64, R=128, inter=0)) == moeq.ESHAPE      # gate/up needs the interleave
    assert sw(r, bank(K=64, R=96)) == moeq.EUNSUPPORTED          # bank rows not a multiple of 64
    assert sw(r, bank(K=64, R=128), act=moeq.F32) == moeq.EUNSUPPORTED
    assert sw(r, bank(K=64, R=128), wsp=0) == moeq.EINVAL
    assert sw(r, bank(K=64, R=128), nbytes=need - 1) == moeq.EWORKSPACE
    dn = lambda w: L.mx8_grouped_down(C.byref(r), P, moeq.BF16, C.byref(w), P, P, need, None)
    assert dn(bank(K=64, R=64, inter=1)) == moeq.ESHAPE
    assert dn(awq()) == moeq.EUNSUPPORTED
