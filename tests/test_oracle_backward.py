"""Oracle backward path (first order): COPY VJP, fixed-selection logit VJP,
combine VJP, SwiGLU VJP and the gate/up + SwiGLU input VJP.

Pins: adjoint identities on exactly representable data (the COPY dispatch, the
combine); an fp32 case whose result depends on the summation order; finite
differences of an independent float64 softmax, of the SwiGLU closed form
(scipy expit) and of the oracle's own forward chain; the two-expert softmax
closed form; values at 0 and beyond the clamp; a linear SwiGLU (alpha = 0)
whose chain VJP is two numpy matmuls with the dense dequantised cubes.
"""
import numpy as np
import pytest
import scipy.special as sp

from quantized_moe_expert_router_amd.synth import CONFIGS, awq_cube, make_inputs


def test_dispatch_backward_adjoint(orc):
    rng = np.random.default_rng(31)
    T, E, k, K = 40, 8, 3, 6
    sel, _ = orc.route(rng.normal(0, 1, (T, E)).astype(np.float32), None, k)
    _, src, pos, _ = orc.dispatch_index(sel, E)
    x = rng.integers(-4, 5, (T, K)).astype(np.float32)
    g = rng.integers(-4, 5, (T * k, K)).astype(np.float32)
    dx = orc.dispatch_backward(g, "f32", pos)
    # <dispatch(x), g> = <x, dispatch_backward(g)>, exact on small integers
    assert np.sum(orc.copy_rows(x, src).astype(np.float64) * g) == np.sum(x * dx.astype(np.float64))
    ref = np.zeros((T, K))
    np.add.at(ref, src, g.astype(np.float64))   # every copy sends its seed back, no weight
    np.testing.assert_array_equal(dx, ref)
    # bf16 storage: the same small integers are exact
    gb = (g.view(np.uint32) >> 16).astype(np.uint16)
    dxb = orc.dispatch_backward(gb, "bf16", pos)
    np.testing.assert_array_equal((dxb.astype(np.uint32) << 16).view(np.float32), ref)


def test_dispatch_backward_sums_in_ascending_expert_order(orc):
    # token 0's slots sit at sorted rows (2, 0, 1); ascending rows: 2^24 + 1 rounds to
    # 2^24, then -2^24 gives 0; summing in slot order would give 1
    pos = np.array([[2, 0, 1]], np.int32)
    g = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], np.float32)
    assert orc.dispatch_backward(g, "f32", pos)[0, 0] == 0.0


def _softmax64(s):
    z = np.exp(s - s.max())
    return z / z.sum()


def test_weights_backward_finite_differences(orc):
    rng = np.random.default_rng(32)
    T, E, k = 25, 16, 4
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    sel, w = orc.route(logits, None, k)
    dw = rng.normal(0, 1, (T, k)).astype(np.float32)
    dl = orc.dispatch_weights_backward(sel, w, dw, E)
    eps = 1e-5
    for t in range(T):
        s = logits[t, sel[t]].astype(np.float64)          # selection held fixed
        for j in range(k):
            d = np.zeros(k)
            d[j] = eps
            fd = (np.dot(dw[t], _softmax64(s + d)) - np.dot(dw[t], _softmax64(s - d))) / (2 * eps)
            assert dl[t, sel[t, j]] == pytest.approx(fd, rel=1e-5, abs=1e-7)
        others = np.setdiff1d(np.arange(E), sel[t])
        assert np.all(dl[t, others] == 0.0)               # a discrete selection: no derivative
        assert abs(float(dl[t].astype(np.float64).sum())) <= 1e-6 * (1 + np.abs(dl[t]).sum())


def test_weights_backward_two_expert_closed_form(orc):
    logits = np.array([[0.3, -1.2, 2.0]], np.float32)
    sel, w = orc.route(logits, None, 2)                   # experts 2 and 0
    dw = np.array([[0.7, -0.4]], np.float32)
    dl = orc.dispatch_weights_backward(sel, w, dw, 3)
    s0, s1 = 2.0, float(np.float32(0.3))
    w0 = sp.expit(s0 - s1)                                 # two-way softmax
    d0 = w0 * (1 - w0) * (0.7 - (-0.4))
    assert dl[0, 2] == pytest.approx(d0, rel=1e-6)
    assert dl[0, 0] == pytest.approx(-d0, rel=1e-6)
    assert dl[0, 1] == 0.0


def test_combine_backward_adjoint_and_exact_differences(orc):
    rng = np.random.default_rng(33)
    T, E, k, K = 30, 8, 3, 7
    sel, _ = orc.route(rng.normal(0, 1, (T, E)).astype(np.float32), None, k)
    _, src, pos, _ = orc.dispatch_index(sel, E)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float32), size=(T, k))
    y = rng.integers(-8, 9, (T * k, K)).astype(np.float32)
    dout = rng.integers(-8, 9, (T, K)).astype(np.float32)
    dy, dw = orc.combine_backward(y, "f32", w, pos, dout)
    out = orc.combine(y, "f32", w, pos).astype(np.float64)
    # dyadic weights and small integers: every product and sum is exact in fp32
    assert np.sum(out * dout) == np.sum(y.astype(np.float64) * dy)
    for t in range(0, T, 7):
        for j in range(k):
            w2 = w.copy()
            w2[t, j] += 1.0
            diff = orc.combine(y, "f32", w2, pos).astype(np.float64) - out
            assert np.sum(diff * dout) == dw[t, j]            # exact finite difference
    # only what is requested is formed
    dy2, dw2 = orc.combine_backward(y, "f32", w, pos, dout, want_dweights=False)
    assert dw2 is None and np.array_equal(dy2, dy)


def test_swiglu_backward_finite_differences(orc):
    rng = np.random.default_rng(34)
    n = 4000
    g = rng.normal(0, 2, n).astype(np.float32)
    u = rng.normal(0, 2, n).astype(np.float32)
    dh = rng.normal(0, 1, n).astype(np.float32)
    for alpha, off in ((1.0, 0.0), (1.702, 1.0)):
        dG, dU = orc.swiglu_backward(g, u, dh, "f32", alpha=alpha, up_offset=off)
        g64, u64, d64 = (a.astype(np.float64) for a in (g, u, dh))

        def h(gg, uu):
            return gg * sp.expit(alpha * gg) * (uu + off)
        eps = 1e-6
        fdg = d64 * (h(g64 + eps, u64) - h(g64 - eps, u64)) / (2 * eps)
        fdu = d64 * (h(g64, u64 + eps) - h(g64, u64 - eps)) / (2 * eps)
        np.testing.assert_allclose(dG, fdg, rtol=2e-6, atol=1e-6)
        np.testing.assert_allclose(dU, fdu, rtol=2e-6, atol=1e-6)


def test_swiglu_backward_special_values(orc):
    g = np.array([0.0, 9.0, -7.5, 7.0, 2.0], np.float32)
    u = np.array([3.0, 1.0, 2.0, -7.0, 8.0], np.float32)
    dh = np.array([2.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    dG, dU = orc.swiglu_backward(g, u, dh, "f32", clamp=7.0)
    assert dG[0] == 2.0 * 3.0 * 0.5 and dU[0] == 0.0      # g = 0: sigmoid(0) = 1/2, g' = 0
    assert dG[1] == 0.0 and dG[2] == 0.0                  # beyond the clamp: no derivative
    assert dU[4] == 0.0 and dG[4] != 0.0
    s7 = sp.expit(7.0)                                     # on the boundary: passed through
    assert dG[3] == pytest.approx(-7.0 * (s7 + 7.0 * s7 * (1 - s7)), rel=1e-7)
    assert dU[3] == pytest.approx(7.0 * s7, rel=1e-7)


def _chain_problem(orc, seed, tokens=6):
    cfg = CONFIGS["tiny"]
    p = make_inputs(cfg, seed=seed, T=tokens)
    sel, _ = orc.route(p["logits"], p["router_bias"], cfg.k)
    _, src, _, rex = orc.dispatch_index(sel, cfg.E)
    values = orc.copy_rows(p["x"], src)
    rng = np.random.default_rng(seed + 1)
    gate = awq_cube(rng, cfg.E, cfg.H, cfg.I, cfg.group, "f16", cfg.scale_lo, cfg.scale_hi, True)
    up = awq_cube(rng, cfg.E, cfg.H, cfg.I, cfg.group, "f16", cfg.scale_lo, cfg.scale_hi, True)
    dh = rng.normal(0, 1, (values.shape[0], cfg.I)).astype(np.float32)
    return cfg, values, rex, gate, up, dh


def test_swiglu_input_backward_finite_differences(orc):
    cfg, v, rex, gate, up, dh = _chain_problem(orc, 35)
    dv = orc.awq_swiglu_input_backward(v, "f32", rex, gate, up, "f16", cfg.group, dh)

    def f(x):
        G = orc.awq_project(x, "f32", rex, *gate[:3], "f16", cfg.group, bias=gate[3])
        U = orc.awq_project(x, "f32", rex, *up[:3], "f16", cfg.group, bias=up[3])
        return np.sum(orc.swiglu(G, U, "f32").astype(np.float64) * dh)
    rng = np.random.default_rng(36)
    for _ in range(3):
        d = rng.normal(0, 1, v.shape)
        eps = 1e-2
        fd = (f((v + eps * d).astype(np.float32)) - f((v - eps * d).astype(np.float32))) / (2 * eps)
        assert np.sum(dv.astype(np.float64) * d) == pytest.approx(fd, rel=2e-3)


def test_swiglu_input_backward_linear_case_is_two_matmuls(orc):
    # alpha = 0: h = (g / 2) (u + off), so dG = dh (u + off) / 2 and dU = dh g / 2
    cfg, v, rex, gate, up, dh = _chain_problem(orc, 37)
    off = 0.25
    dv = orc.awq_swiglu_input_backward(v, "f32", rex, gate, up, "f16", cfg.group, dh,
                                       alpha=0.0, up_offset=off).astype(np.float64)
    G = orc.awq_project(v, "f32", rex, *gate[:3], "f16", cfg.group, bias=gate[3]).astype(np.float64)
    U = orc.awq_project(v, "f32", rex, *up[:3], "f16", cfg.group, bias=up[3]).astype(np.float64)
    dG = (dh * (U + off) / 2).astype(np.float32).astype(np.float64)
    dU = (dh * G / 2).astype(np.float32).astype(np.float64)
    Wg = orc.awq_dequant(*gate[:3], "f16", cfg.group)
    Wu = orc.awq_dequant(*up[:3], "f16", cfg.group)
    ref = np.stack([dG[p] @ Wg[rex[p]].T + dU[p] @ Wu[rex[p]].T for p in range(v.shape[0])])
    np.testing.assert_allclose(dv, ref, rtol=1e-6, atol=1e-6)


def test_swiglu_one_sided_gate_clamp(orc):
    """The variant some MXFP4 models use (gate clamped from above only, alpha 1.702,
    up + 1): closed form in float64, and its derivatives by central differences."""
    c, alpha, off = 7.0, 1.702, 1.0
    g = np.array([-20.0, -7.5, -3.0, 0.0, 3.0, 7.0, 9.0, -9.0], np.float32)
    u = np.array([2.0, -9.0, 8.0, 1.0, -2.0, 3.0, 0.5, -6.0], np.float32)
    h = orc.swiglu(g, u, "f32", clamp=c, alpha=alpha, up_offset=off, gate_one_sided=True)
    gp = np.minimum(g.astype(np.float64), c)
    up = np.clip(u.astype(np.float64), -c, c)
    ref = gp * sp.expit(alpha * gp) * (up + off)
    np.testing.assert_allclose(h, ref, rtol=1e-6, atol=1e-30)
    two = orc.swiglu(g, u, "f32", clamp=c, alpha=alpha, up_offset=off)
    assert h[0] != two[0] and h[3] == two[3]      # only the gate's lower clamp differs
    d = np.ones_like(g)
    dG, dU = orc.swiglu_backward(g, u, d, "f32", clamp=c, alpha=alpha, up_offset=off,
                                 gate_one_sided=True)
    eps = 1e-6

    def hf(gg, uu):
        gg, uu = np.minimum(gg, c), np.clip(uu, -c, c)
        return gg * sp.expit(alpha * gg) * (uu + off)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    inside = g64 < c - 1e-3                                   # away from the kink at c
    fdg = (hf(g64 + eps, u64) - hf(g64 - eps, u64)) / (2 * eps)
    np.testing.assert_allclose(dG[inside], fdg[inside], rtol=1e-5, atol=1e-7)
    assert dG[6] == 0.0 and dG[0] != 0.0                      # above c: blocked; below -c: not
    assert dU[1] == 0.0                                       # u beyond the clamp: blocked
