"""Pins of the oracle's MXFP4 expert-bank composition.

The bank layout is the one libmir-metal 0.3.0's native.rs describes
(ExpertLayout::Native, `native_layout` with an interleaved FusedGateUpBank,
`validate` with companion shapes blocks [E, 2I, H/32, 16], scales [E, 2I, H/32],
bias [E, 2I]; the down bank [E, H, I/32, 16] with bias [E, H]).  Readings the
pages leave open: row 2i of the fused bank is gate feature i and row 2i+1 is up
feature i, with the bias interleaved the same way; the clamped SwiGLU clamps both
halves to [-c, c] (the "clamped_routed" engine).

What pins the oracle here, independently of its own code:
  * the dense banks are built by this file from the golden E2M1 / E8M0 tables
    (tests/golden/mxfp4.txt), never through the oracle's decoder;
  * separate gate and up banks are interleaved here, so a gate/up swap or a
    different interleave granularity in the oracle fails;
  * every bias is non-zero and differs per expert and per row, so a bias indexed
    without the expert fails;
  * the whole path is evaluated per token in float64 with no dispatch or sort.
"""
import numpy as np
import pytest
import scipy.special as sp

from conftest import read_golden


def golden_tables():
    e2m1 = np.zeros(16)
    for row in read_golden("mxfp4.txt"):
        if row[0] == "e2m1":
            e2m1[int(row[1])] = float(row[2])
    return e2m1


def dense_bank(blocks, scales):
    """blocks u8 [E, R, C/32, 16], scales u8 [E, R, C/32] -> float64 [E, R, C]."""
    table = golden_tables()
    E, R, NB, _ = blocks.shape
    lo, hi = blocks & 0xF, blocks >> 4                    # even element in the low nibble
    elems = np.stack([lo, hi], -1).reshape(E, R, NB, 32)
    scale = 2.0 ** (scales.astype(np.float64) - 127.0)
    return (table[elems] * scale[..., None]).reshape(E, R, NB * 32)


def interleave_rows(gate, up):
    """Two arrays [E, I, ...] -> [E, 2I, ...] with gate row i at 2i, up row i at 2i+1."""
    E, I = gate.shape[:2]
    return np.stack([gate, up], axis=2).reshape(E, 2 * I, *gate.shape[2:])


def bf16_bits(v):
    """float64 -> bf16 bit patterns, one round to nearest even at 8 significant
    bits (the values here are normal and finite)."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.round(np.ldexp(m, 8)), e - 8)        # np.round: ties to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_values(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def small_bank_inputs(seed, T=12, H=64, I=32, E=4, k=2, adt="f32", clamp=7.0):
    rng = np.random.default_rng(seed)
    g_blocks = rng.integers(0, 256, (E, I, H // 32, 16), dtype=np.uint8)
    u_blocks = rng.integers(0, 256, (E, I, H // 32, 16), dtype=np.uint8)
    g_scales = rng.integers(122, 128, (E, I, H // 32), dtype=np.uint8)
    u_scales = rng.integers(122, 128, (E, I, H // 32), dtype=np.uint8)
    # biases on the order of the products, different per expert and per row
    g_bias = bf16_bits(rng.normal(0.0, 2.0, (E, I)))
    u_bias = bf16_bits(rng.normal(0.0, 2.0, (E, I)))
    x = rng.normal(0.0, 1.0, (T, H)).astype(np.float32)
    if adt == "bf16":
        x = bf16_bits(x)
    p = dict(fmt="mxfp4", T=T, H=H, I=I, E=E, k=k, group=32, adt=adt, sdt="bf16",
             clamp=clamp, alpha=1.0, up_offset=0.0, x=x,
             logits=rng.normal(0.0, 1.0, (T, E)).astype(np.float32), router_bias=None,
             gu_blocks=interleave_rows(g_blocks, u_blocks),
             gu_scales=interleave_rows(g_scales, u_scales),
             gu_bias=interleave_rows(g_bias, u_bias),
             dn_blocks=rng.integers(0, 256, (E, H, I // 32, 16), dtype=np.uint8),
             dn_scales=rng.integers(122, 128, (E, H, I // 32), dtype=np.uint8),
             dn_bias=bf16_bits(rng.normal(0.0, 2.0, (E, H))))
    sep = dict(g_blocks=g_blocks, u_blocks=u_blocks, g_scales=g_scales, u_scales=u_scales,
               g_bias=g_bias, u_bias=u_bias)
    return p, sep


def test_interleave_round_trip():
    rng = np.random.default_rng(40)
    g = rng.integers(0, 256, (3, 5, 2, 16), dtype=np.uint8)
    u = rng.integers(0, 256, (3, 5, 2, 16), dtype=np.uint8)
    b = interleave_rows(g, u)
    assert b.shape == (3, 10, 2, 16)
    np.testing.assert_array_equal(b[:, 0::2], g)
    np.testing.assert_array_equal(b[:, 1::2], u)
    # a one-row-per-expert case spelled out by hand
    g1, u1 = np.array([[7], [9]]), np.array([[8], [10]])
    np.testing.assert_array_equal(interleave_rows(g1[:, :, None], u1[:, :, None])[..., 0],
                                  [[7, 8], [9, 10]])


def test_mxfp4_project_bias_is_per_expert_and_row(orc):
    """Exact arithmetic: integer activations and power-of-two scales keep every
    product and partial sum exact, so the oracle must match the dense float64
    product plus bias[e, r] bit for bit.  A bias read as bias[r] (without the
    expert) or as bias[e] would fail."""
    rng = np.random.default_rng(41)
    E, R, Cin, A = 4, 24, 64, 40
    blocks = rng.integers(0, 256, (E, R, Cin // 32, 16), dtype=np.uint8)
    scales = rng.integers(124, 129, (E, R, Cin // 32), dtype=np.uint8)
    W = dense_bank(blocks, scales)
    # bias values are small dyadic numbers, exact in bf16 and distinct per (e, r)
    bias_vals = (np.arange(E * R).reshape(E, R) - E * R / 2) / 8.0
    bias = bf16_bits(bias_vals)
    np.testing.assert_array_equal(bf16_values(bias), bias_vals)
    x = rng.integers(-2, 3, (A, Cin)).astype(np.float32)
    rex = np.sort(rng.integers(0, E, A)).astype(np.uint32)
    out = orc.mxfp4_project(x, "f32", rex, blocks, scales, bias)
    ref = np.stack([W[rex[p]] @ x[p].astype(np.float64) + bias_vals[rex[p]] for p in range(A)])
    np.testing.assert_array_equal(out.astype(np.float64), ref)
    # the planted alternatives differ from the oracle's result
    wrong = np.stack([W[rex[p]] @ x[p].astype(np.float64) + bias_vals[0] for p in range(A)])
    assert not np.array_equal(out.astype(np.float64), wrong)


def test_mxfp4_project_separate_banks_equal_interleaved(orc):
    """Projecting with the fused bank equals projecting with the gate and up banks
    on their own, row 2i <- gate i and row 2i+1 <- up i, bit for bit."""
    p, sep = small_bank_inputs(42, adt="bf16")
    A = 30
    rng = np.random.default_rng(43)
    x = bf16_bits(rng.normal(0, 1, (A, p["H"])))
    rex = np.sort(rng.integers(0, p["E"], A)).astype(np.uint32)
    fused = orc.mxfp4_project(x, "bf16", rex, p["gu_blocks"], p["gu_scales"], p["gu_bias"])
    g = orc.mxfp4_project(x, "bf16", rex, sep["g_blocks"], sep["g_scales"], sep["g_bias"])
    u = orc.mxfp4_project(x, "bf16", rex, sep["u_blocks"], sep["u_scales"], sep["u_bias"])
    np.testing.assert_array_equal(fused[:, 0::2], g)
    np.testing.assert_array_equal(fused[:, 1::2], u)


def dense_bank_forward(orc, p, sep, one_sided=False):
    """Per-token float64 evaluation of the clamped-SwiGLU MXFP4 path, with no
    dispatch: out[t] = sum over t's experts in ascending ID of w * FFN_e(x_t), with
    the storage roundings (to the activation type) at G, U, h and Y."""
    T, E, k = p["T"], p["E"], p["k"]
    adt = p["adt"]
    sel, w = orc.route(p["logits"], p["router_bias"], k)
    Wg = dense_bank(sep["g_blocks"], sep["g_scales"])
    Wu = dense_bank(sep["u_blocks"], sep["u_scales"])
    Wd = dense_bank(p["dn_blocks"], p["dn_scales"])
    bg, bu, bd = bf16_values(sep["g_bias"]), bf16_values(sep["u_bias"]), bf16_values(p["dn_bias"])
    if adt == "f32":
        rnd = lambda a: np.asarray(a).astype(np.float32).astype(np.float64)
        x = p["x"].astype(np.float64)
    else:
        rnd = lambda a: bf16_values(bf16_bits(a))
        x = bf16_values(p["x"])
    c, alpha, off = p["clamp"], p["alpha"], p["up_offset"]
    out = np.zeros((T, p["H"]))
    stats = []
    for t in range(T):
        for j in np.argsort(sel[t]):                       # ascending expert ID
            e = sel[t, j]
            G = rnd(Wg[e] @ x[t] + bg[e])
            U = rnd(Wu[e] @ x[t] + bu[e])
            stats.append((np.mean(np.abs(G) > c), np.mean(np.abs(U) > c)))
            g = np.minimum(G, c) if one_sided else np.clip(G, -c, c)
            u = np.clip(U, -c, c)
            h = rnd(g * sp.expit(alpha * g) * (u + off))
            y = rnd(Wd[e] @ h + bd[e])
            out[t] += float(w[t, j]) * y
    return out, np.array(stats)


@pytest.mark.parametrize("adt", ["f32", "bf16"])
def test_forward_mxfp4_against_dense(orc, adt):
    p, sep = small_bank_inputs(44, adt=adt)
    res = orc.moe_forward(p)
    ref, stats = dense_bank_forward(orc, p, sep)
    # the clamp is active on part, not all, of G and U, so it is exercised
    assert 0.05 < stats[:, 0].mean() < 0.95 and 0.05 < stats[:, 1].mean() < 0.95
    if adt == "f32":
        got = res["out"].astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    else:
        got = bf16_values(res["out"])
        den = np.max(np.abs(ref), axis=1)
        assert np.max(np.max(np.abs(got - ref), axis=1) / den) < 1e-2
    # a gate/up swap would be far outside the tolerance
    p_sw = dict(p, gu_blocks=interleave_rows(sep["u_blocks"], sep["g_blocks"]),
                gu_scales=interleave_rows(sep["u_scales"], sep["g_scales"]),
                gu_bias=interleave_rows(sep["u_bias"], sep["g_bias"]))
    swapped = orc.moe_forward(p_sw)["out"]
    swapped = swapped.astype(np.float64) if adt == "f32" else bf16_values(swapped)
    assert np.max(np.abs(swapped - ref)) > 10 * np.max(np.abs(got - ref)) + 1e-3


def test_forward_mxfp4_one_sided_against_dense(orc):
    p, sep = small_bank_inputs(45, adt="f32")
    p.update(alpha=1.702, up_offset=1.0, gate_one_sided=True)
    res = orc.moe_forward(p)
    ref, _ = dense_bank_forward(orc, p, sep, one_sided=True)
    np.testing.assert_allclose(res["out"].astype(np.float64), ref, rtol=1e-5,
                               atol=1e-5 * np.abs(ref).max())


def test_forward_mxfp4_intermediates(orc):
    """The oracle's G/U split, SwiGLU and down bank, step by step: h equals the
    clamped SwiGLU of the two separately projected banks, and y the down bank's
    projection of h, bit for bit."""
    p, sep = small_bank_inputs(46, adt="bf16")
    res = orc.moe_forward(p)
    rex, values = res["row_experts"], res["values"]
    G = orc.mxfp4_project(values, "bf16", rex, sep["g_blocks"], sep["g_scales"], sep["g_bias"])
    U = orc.mxfp4_project(values, "bf16", rex, sep["u_blocks"], sep["u_scales"], sep["u_bias"])
    np.testing.assert_array_equal(res["h"], orc.swiglu(G, U, "bf16", clamp=p["clamp"]))
    y = orc.mxfp4_project(res["h"], "bf16", rex, p["dn_blocks"], p["dn_scales"], p["dn_bias"])
    np.testing.assert_array_equal(res["y"], y)
    # and the down projection with the dense bank from the golden tables
    Wd = dense_bank(p["dn_blocks"], p["dn_scales"])
    hv = bf16_values(res["h"])
    yd = np.stack([Wd[e] @ hv[i] for i, e in enumerate(rex)]) + bf16_values(p["dn_bias"])[rex]
    np.testing.assert_array_equal(bf16_values(res["y"]), bf16_values(bf16_bits(yd)))
