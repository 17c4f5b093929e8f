"""Plain CPU oracle for the routed MoE expert FFN (numpy front end over moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library and never imports it.

Storage conventions: ``"f32"`` arrays are ``float32``, ``"f16"`` arrays are
``float16``, ``"bf16"`` arrays are ``uint16`` bit patterns.  Packed AWQ words are
``int32``, MXFP4 blocks and scales ``uint8``.

The per-function citations and what pins each function are in moe_oracle.c.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SANITIZE = os.environ.get("MOEQ_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle_san.so" if _SANITIZE else "libmoe_oracle.so")
_lib = None

DT = {"f32": 0, "f16": 1, "bf16": 2}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build(sanitize=_SANITIZE)
    lib = C.CDLL(_LIB_PATH)
    vp, i32, u32p = C.c_void_p, C.c_int, C.c_void_p
    lib.orc_round_f16.restype = C.c_uint16
    lib.orc_round_f16.argtypes = [C.c_double]
    lib.orc_round_bf16.restype = C.c_uint16
    lib.orc_round_bf16.argtypes = [C.c_double]
    lib.orc_f16_value.restype = C.c_double
    lib.orc_f16_value.argtypes = [C.c_uint16]
    lib.orc_bf16_value.restype = C.c_double
    lib.orc_bf16_value.argtypes = [C.c_uint16]
    lib.orc_route.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.orc_dispatch_index.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.orc_copy_rows.argtypes = [i32, C.c_size_t, vp, vp, vp]
    lib.orc_counts.restype = C.c_int
    lib.orc_counts.argtypes = [i32, vp, i32, vp, vp]
    lib.orc_awq_coeff.restype = C.c_double
    lib.orc_awq_coeff.argtypes = [i32, i32, i32, vp, vp, vp, i32, i32, i32, i32]
    lib.orc_awq_dequant.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp]
    lib.orc_awq_project.argtypes = [i32, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp, i32,
                                    vp, vp, vp]
    lib.orc_swiglu.argtypes = [C.c_size_t, vp, vp, i32, C.c_double, C.c_double, C.c_double,
                               i32, vp]
    lib.orc_combine.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
    lib.orc_copy_vjp.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.orc_awq_input_backward.argtypes = [i32, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp,
                                           i32, vp]
    lib.orc_dispatch_backward.argtypes = [i32, i32, i32, vp, i32, vp, vp]
    lib.orc_dispatch_weights_backward.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.orc_combine_backward.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.orc_swiglu_backward.argtypes = [C.c_size_t, vp, vp, vp, i32, C.c_double, C.c_double,
                                        C.c_double, i32, vp, vp]
    lib.orc_awq_swiglu_input_backward.argtypes = [i32, i32, i32, vp, i32, vp, i32, i32,
                                                  vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                                  C.c_double, C.c_double, C.c_double, i32,
                                                  vp, vp]
    lib.orc_e2m1_value.restype = C.c_double
    lib.orc_e2m1_value.argtypes = [i32]
    lib.orc_e8m0_value.restype = C.c_double
    lib.orc_e8m0_value.argtypes = [i32]
    lib.orc_mxfp4_dequant.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.orc_mxfp4_project.argtypes = [i32, i32, i32, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.orc_e4m3_value.restype = C.c_double
    lib.orc_e4m3_value.argtypes = [i32]
    lib.orc_mxfp8_quantize.argtypes = [i32, i32, vp, i32, vp, vp]
    lib.orc_mx8_project.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, i32, vp]
    lib.orc_moe_forward.restype = C.c_int
    lib.orc_moe_forward.argtypes = [vp]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _store(a, dt):
    return np.ascontiguousarray(a, dtype=NP_STORAGE[dt])


# ---------------------------------------------------------------- scalars
def round_f16_bits(v: float) -> int:
    return int(_load().orc_round_f16(float(v)))


def round_bf16_bits(v: float) -> int:
    return int(_load().orc_round_bf16(float(v)))


def f16_value(bits: int) -> float:
    return float(_load().orc_f16_value(int(bits)))


def bf16_value(bits: int) -> float:
    return float(_load().orc_bf16_value(int(bits)))


def e2m1_value(nibble: int) -> float:
    return float(_load().orc_e2m1_value(int(nibble)))


def e8m0_value(byte: int) -> float:
    return float(_load().orc_e8m0_value(int(byte)))


# ---------------------------------------------------------------- routing
def route(logits, bias, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    sel = np.zeros((T, k), np.uint32)
    w = np.zeros((T, k), np.float32)
    _load().orc_route(T, E, k, _p(logits), _p(b), _p(sel), _p(w))
    return sel, w


def dispatch_index(selected, E):
    selected = _c(selected, np.uint32)
    T, k = selected.shape
    A = T * k
    off = np.zeros(E + 1, np.int32)
    src = np.zeros(A, np.int32)
    pos = np.zeros((T, k), np.int32)
    rex = np.zeros(A, np.uint32)
    _load().orc_dispatch_index(T, E, k, _p(selected), _p(off), _p(src), _p(pos), _p(rex))
    return off, src, pos, rex


def copy_rows(x, row_src):
    x = np.ascontiguousarray(x)
    row_src = _c(row_src, np.int32)
    A = row_src.shape[0]
    out = np.zeros((A,) + x.shape[1:], x.dtype)
    row_bytes = x[0].nbytes if x.shape[0] else 0
    _load().orc_copy_rows(A, row_bytes, _p(x), _p(row_src), _p(out))
    return out


def counts(offsets, prefix):
    offsets = _c(offsets, np.int32)
    prefix = _c(prefix, np.int64)
    R = prefix.shape[0] - 1
    out = np.zeros(max(R, 0), np.int64)
    rc = _load().orc_counts(offsets.shape[0] - 1, _p(offsets), R, _p(prefix), _p(out))
    if rc != 0:
        raise ValueError("invalid expert prefix")
    return out


# ---------------------------------------------------------------- AWQ
def awq_coeff(qweight, qzeros, scales, sdt, g, e, k, n):
    qweight = _c(qweight, np.int32)
    qzeros = _c(qzeros, np.int32)
    scales = _store(scales, sdt)
    E, K, W8 = qweight.shape
    return float(_load().orc_awq_coeff(K, W8 * 8, g, _p(qweight), _p(qzeros), _p(scales),
                                       DT[sdt], e, k, n))


def awq_dequant(qweight, qzeros, scales, sdt, g):
    qweight = _c(qweight, np.int32)
    qzeros = _c(qzeros, np.int32)
    scales = _store(scales, sdt)
    E, K, W8 = qweight.shape
    N = W8 * 8
    W = np.zeros((E, K, N), np.float64)
    _load().orc_awq_dequant(E, K, N, g, _p(qweight), _p(qzeros), _p(scales), DT[sdt], _p(W))
    return W


def awq_project(x, adt, row_experts, qweight, qzeros, scales, sdt, g, bias=None,
                want_exact=False):
    x = _store(x, adt)
    A, K = x.shape
    qweight = _c(qweight, np.int32)
    qzeros = _c(qzeros, np.int32)
    scales = _store(scales, sdt)
    E, K2, W8 = qweight.shape
    assert K2 == K
    N = W8 * 8
    rex = None if row_experts is None else _c(row_experts, np.uint32)
    b = None if bias is None else _store(bias, sdt)
    out = np.zeros((A, N), NP_STORAGE[adt])
    exact = np.zeros((A, N), np.float64) if want_exact else None
    _load().orc_awq_project(A, K, N, _p(x), DT[adt], _p(rex), E, g, _p(qweight), _p(qzeros),
                            _p(scales), DT[sdt], _p(b), _p(out), _p(exact))
    return (out, exact) if want_exact else out


def swiglu(G, U, adt, clamp=0.0, alpha=1.0, up_offset=0.0, gate_one_sided=False):
    G = _store(G, adt)
    U = _store(U, adt)
    h = np.zeros_like(G)
    _load().orc_swiglu(G.size, _p(G), _p(U), DT[adt], float(clamp), float(alpha),
                       float(up_offset), int(bool(gate_one_sided)), _p(h))
    return h


def combine(y, adt, weights, slot_pos):
    y = _store(y, adt)
    weights = _c(weights, np.float32)
    slot_pos = _c(slot_pos, np.int32)
    T, k = slot_pos.shape
    K = y.shape[1]
    out = np.zeros((T, K), NP_STORAGE[adt])
    _load().orc_combine(T, k, K, _p(y), DT[adt], _p(weights), _p(slot_pos), _p(out))
    return out


def copy_vjp(dvalues, slot_pos):
    dvalues = _c(dvalues, np.float64)
    slot_pos = _c(slot_pos, np.int32)
    T, k = slot_pos.shape
    K = dvalues.shape[1]
    dx = np.zeros((T, K), np.float64)
    _load().orc_copy_vjp(T, k, K, _p(dvalues), _p(slot_pos), _p(dx))
    return dx


def awq_input_backward(grad, gdt, row_experts, qweight, qzeros, scales, sdt, g):
    grad = _store(grad, gdt)
    A, N = grad.shape
    qweight = _c(qweight, np.int32)
    qzeros = _c(qzeros, np.int32)
    scales = _store(scales, sdt)
    E, K, W8 = qweight.shape
    assert W8 * 8 == N
    rex = None if row_experts is None else _c(row_experts, np.uint32)
    out = np.zeros((A, K), NP_STORAGE[gdt])
    _load().orc_awq_input_backward(A, K, N, _p(grad), DT[gdt], _p(rex), E, g, _p(qweight),
                                   _p(qzeros), _p(scales), DT[sdt], _p(out))
    return out


# ---------------------------------------------------------------- backward path
def dispatch_backward(dvalues, adt, slot_pos):
    """COPY VJP: dx[t] = round_adt(fp32 sum of the token's gradient rows in
    ascending sorted position)."""
    dvalues = _store(dvalues, adt)
    slot_pos = _c(slot_pos, np.int32)
    T, k = slot_pos.shape
    K = dvalues.shape[1]
    dx = np.zeros((T, K), NP_STORAGE[adt])
    _load().orc_dispatch_backward(T, k, K, _p(dvalues), DT[adt], _p(slot_pos), _p(dx))
    return dx


def dispatch_weights_backward(selected, weights, dweights, E):
    """Fixed-selection logit VJP of the softmax weights: dlogits [T, E] fp32."""
    selected = _c(selected, np.uint32)
    weights = _c(weights, np.float32)
    dweights = _c(dweights, np.float32)
    T, k = selected.shape
    dl = np.zeros((T, E), np.float32)
    _load().orc_dispatch_weights_backward(T, E, k, _p(selected), _p(weights), _p(dweights),
                                          _p(dl))
    return dl


def combine_backward(y, adt, weights, slot_pos, dout, want_dy=True, want_dweights=True):
    """Combine VJP: (dy [A, K] adt or None, dweights [T, k] fp32 or None)."""
    y = _store(y, adt)
    weights = _c(weights, np.float32)
    slot_pos = _c(slot_pos, np.int32)
    dout = _store(dout, adt)
    T, k = slot_pos.shape
    K = y.shape[1]
    dy = np.zeros_like(y) if want_dy else None
    dw = np.zeros((T, k), np.float32) if want_dweights else None
    _load().orc_combine_backward(T, k, K, _p(y), DT[adt], _p(weights), _p(slot_pos), _p(dout),
                                 _p(dy), _p(dw))
    return dy, dw


def swiglu_backward(G, U, dh, adt, clamp=0.0, alpha=1.0, up_offset=0.0, gate_one_sided=False):
    """SwiGLU VJP at the forward's storage-rounded G, U: (dG, dU) in adt."""
    G = _store(G, adt)
    U = _store(U, adt)
    dh = _store(dh, adt)
    dG = np.zeros_like(G)
    dU = np.zeros_like(G)
    _load().orc_swiglu_backward(G.size, _p(G), _p(U), _p(dh), DT[adt], float(clamp),
                                float(alpha), float(up_offset), int(bool(gate_one_sided)),
                                _p(dG), _p(dU))
    return dG, dU


def awq_swiglu_input_backward(values, adt, row_experts, gate, up, sdt, g, dh, clamp=0.0,
                              alpha=1.0, up_offset=0.0, gate_one_sided=False):
    """Input VJP of the gate/up + SwiGLU part: dvalues [A, K] adt.
    gate / up: (qweight, qzeros, scales, bias or None) of equal shape."""
    values = _store(values, adt)
    A, K = values.shape
    gqw, gqz, gs, gb = gate
    uqw, uqz, us, ub = up
    gqw, uqw = _c(gqw, np.int32), _c(uqw, np.int32)
    gqz, uqz = _c(gqz, np.int32), _c(uqz, np.int32)
    gs, us = _store(gs, sdt), _store(us, sdt)
    gb = None if gb is None else _store(gb, sdt)
    ub = None if ub is None else _store(ub, sdt)
    E, K2, W8 = gqw.shape
    assert K2 == K
    I = W8 * 8
    dh = _store(dh, adt)
    rex = None if row_experts is None else _c(row_experts, np.uint32)
    out = np.zeros((A, K), NP_STORAGE[adt])
    _load().orc_awq_swiglu_input_backward(A, K, I, _p(values), DT[adt], _p(rex), E, g,
                                          _p(gqw), _p(gqz), _p(gs), _p(uqw), _p(uqz), _p(us),
                                          DT[sdt], _p(gb), _p(ub), float(clamp), float(alpha),
                                          float(up_offset), int(bool(gate_one_sided)), _p(dh),
                                          _p(out))
    return out


# ---------------------------------------------------------------- MXFP4
def mxfp4_dequant(blocks, scales):
    blocks = _c(blocks, np.uint8)
    scales = _c(scales, np.uint8)
    E, R, NB, sixteen = blocks.shape
    assert sixteen == 16 and scales.shape == (E, R, NB)
    W = np.zeros((E, R, NB * 32), np.float64)
    _load().orc_mxfp4_dequant(E, R, NB * 32, _p(blocks), _p(scales), _p(W))
    return W


def mxfp4_project(x, adt, row_experts, blocks, scales, bias_bf16):
    x = _store(x, adt)
    A, Cin = x.shape
    blocks = _c(blocks, np.uint8)
    scales = _c(scales, np.uint8)
    E, R, NB, _ = blocks.shape
    assert NB * 32 == Cin
    rex = None if row_experts is None else _c(row_experts, np.uint32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    out = np.zeros((A, R), NP_STORAGE[adt])
    _load().orc_mxfp4_project(A, Cin, R, _p(x), DT[adt], _p(rex), E, _p(blocks), _p(scales),
                              _p(b), _p(out))
    return out


# ---------------------------------------------------------------- MXFP8 activations
def e4m3_value(byte: int) -> float:
    return float(_load().orc_e4m3_value(int(byte)))


def mxfp8_quantize(x, adt):
    """OCP MX quantization of 32-element row blocks: (codes u8 [rows, K], scales u8 [rows, K/32])."""
    x = _store(x, adt)
    rows, K = x.shape
    q = np.zeros((rows, K), np.uint8)
    s = np.zeros((rows, K // 32), np.uint8)
    _load().orc_mxfp8_quantize(rows, K, _p(x), DT[adt], _p(q), _p(s))
    return q, s


def mx8_project(q, s, row_experts, blocks, scales, bias_bf16, adt):
    """Projection of MXFP8 rows with an MXFP4 bank, output rounded to adt."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    blocks = _c(blocks, np.uint8)
    scales = _c(scales, np.uint8)
    E, R, NB, sixteen = blocks.shape
    A, C_ = q.shape
    assert NB * 32 == C_
    rex = None if row_experts is None else _c(row_experts, np.uint32)
    b = None if bias_bf16 is None else _c(bias_bf16, np.uint16)
    out = np.zeros((A, R), NP_STORAGE[adt])
    _load().orc_mx8_project(A, C_, R, _p(q), _p(s), _p(rex), E, _p(blocks), _p(scales), _p(b),
                            DT[adt], _p(out))
    return out


# ---------------------------------------------------------------- whole path
class _MoeArgs(C.Structure):
    _fields_ = [
        ("fmt", C.c_int), ("T", C.c_int), ("H", C.c_int), ("I", C.c_int), ("E", C.c_int),
        ("k", C.c_int), ("group", C.c_int), ("adt", C.c_int), ("sdt", C.c_int),
        ("x", C.c_void_p), ("logits", C.c_void_p), ("router_bias", C.c_void_p),
        ("gate_qw", C.c_void_p), ("gate_qz", C.c_void_p), ("up_qw", C.c_void_p),
        ("up_qz", C.c_void_p), ("down_qw", C.c_void_p), ("down_qz", C.c_void_p),
        ("gate_s", C.c_void_p), ("up_s", C.c_void_p), ("down_s", C.c_void_p),
        ("gate_b", C.c_void_p), ("up_b", C.c_void_p), ("down_b", C.c_void_p),
        ("gu_blocks", C.c_void_p), ("gu_scales", C.c_void_p), ("dn_blocks", C.c_void_p),
        ("dn_scales", C.c_void_p), ("gu_bias", C.c_void_p), ("dn_bias", C.c_void_p),
        ("clamp", C.c_double), ("alpha", C.c_double), ("up_offset", C.c_double),
        ("gate_one_sided", C.c_int), ("out", C.c_void_p),
        ("selected", C.c_void_p), ("weights", C.c_void_p), ("offsets", C.c_void_p),
        ("row_src", C.c_void_p), ("slot_pos", C.c_void_p), ("row_experts", C.c_void_p),
        ("values", C.c_void_p), ("h", C.c_void_p), ("y", C.c_void_p),
    ]


def moe_forward(p: dict, keep_intermediates: bool = True) -> dict:
    """Whole path logits -> out on the inputs dict produced by the seeded generator.

    Keys used: fmt ("awq"|"mxfp4"), T, H, I, E, k, group, adt, sdt, x, logits,
    router_bias, and the weight arrays (gate_qw/... or gu_blocks/...), clamp,
    alpha, up_offset.
    """
    lib = _load()
    T, H, I, E, k = p["T"], p["H"], p["I"], p["E"], p["k"]
    adt, sdt = p["adt"], p.get("sdt", "bf16")
    A = T * k
    keep = []

    def ptr(a, dtype=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a) if dtype is None else np.ascontiguousarray(a, dtype)
        keep.append(a)
        return a.ctypes.data_as(C.c_void_p).value

    args = _MoeArgs()
    args.fmt = 0 if p["fmt"] == "awq" else 1
    args.T, args.H, args.I, args.E, args.k = T, H, I, E, k
    args.group = p.get("group", 32)
    args.adt, args.sdt = DT[adt], DT[sdt]
    args.x = ptr(_store(p["x"], adt))
    args.logits = ptr(p["logits"], np.float32)
    args.router_bias = ptr(p.get("router_bias"), np.float32)
    if p["fmt"] == "awq":
        for nm in ("gate", "up", "down"):
            setattr(args, nm + "_qw", ptr(p[nm + "_qw"], np.int32))
            setattr(args, nm + "_qz", ptr(p[nm + "_qz"], np.int32))
            setattr(args, nm + "_s", ptr(_store(p[nm + "_s"], sdt)))
            b = p.get(nm + "_b")
            setattr(args, nm + "_b", ptr(None if b is None else _store(b, sdt)))
    else:
        args.gu_blocks = ptr(p["gu_blocks"], np.uint8)
        args.gu_scales = ptr(p["gu_scales"], np.uint8)
        args.dn_blocks = ptr(p["dn_blocks"], np.uint8)
        args.dn_scales = ptr(p["dn_scales"], np.uint8)
        args.gu_bias = ptr(p["gu_bias"], np.uint16)
        args.dn_bias = ptr(p["dn_bias"], np.uint16)
    args.clamp = float(p.get("clamp", 0.0))
    args.alpha = float(p.get("alpha", 1.0))
    args.up_offset = float(p.get("up_offset", 0.0))
    args.gate_one_sided = int(bool(p.get("gate_one_sided", False)))
    st = NP_STORAGE[adt]
    res = {"out": np.zeros((T, H), st)}
    args.out = res["out"].ctypes.data_as(C.c_void_p).value
    if keep_intermediates:
        res.update(selected=np.zeros((T, k), np.uint32), weights=np.zeros((T, k), np.float32),
                   offsets=np.zeros(E + 1, np.int32), row_src=np.zeros(A, np.int32),
                   slot_pos=np.zeros((T, k), np.int32), row_experts=np.zeros(A, np.uint32),
                   values=np.zeros((A, H), st), h=np.zeros((A, I), st), y=np.zeros((A, H), st))
        for nm in ("selected", "weights", "offsets", "row_src", "slot_pos", "row_experts",
                   "values", "h", "y"):
            setattr(args, nm, res[nm].ctypes.data_as(C.c_void_p).value)
    rc = lib.orc_moe_forward(C.byref(args))
    assert rc == 0
    del keep
    return res
