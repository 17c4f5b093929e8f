"""Oracle router (top-k + FP32 softmax) and COPY dispatch against brute force.

Pins: numpy lexsort over (score desc, id asc); scipy softmax / expit; closed-form
cases; numpy stable argsort and bincount for the dispatch order.
"""
import numpy as np
import pytest
import scipy.special as sp


def brute_topk(scores, k):
    T, E = scores.shape
    out = np.zeros((T, k), np.uint32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -scores[t].astype(np.float64)))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("T,E,k,grid", [(37, 8, 2, None), (50, 128, 8, None),
                                         (40, 512, 10, None), (64, 16, 4, 1.0),
                                         (64, 128, 8, 0.5), (9, 5, 5, None), (3, 7, 1, None)])
def test_topk_brute_force(orc, T, E, k, grid):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    if grid is not None:   # coarse grid: many exact ties
        logits = (np.round(logits / grid) * grid).astype(np.float32)
    sel, w = orc.route(logits, None, k)
    np.testing.assert_array_equal(sel, brute_topk(logits, k))
    chosen = np.take_along_axis(logits.astype(np.float64), sel.astype(np.int64), 1)
    ref = sp.softmax(chosen, axis=1).astype(np.float32)
    np.testing.assert_allclose(w, ref, rtol=2e-7, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)          # slots in descending score
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=k * 2.0 ** -24)


def test_bias_is_added_before_selection(orc):
    logits = np.array([[1.0, 0.9, 0.0, -1.0]], np.float32)
    bias = np.array([0.0, 0.5, 0.0, 3.0], np.float32)
    sel, w = orc.route(logits, bias, 2)
    assert sel.tolist() == [[3, 1]]
    s = (logits + bias)[0]
    np.testing.assert_allclose(w[0], sp.softmax(s[[3, 1]].astype(np.float64)), rtol=2e-7)
    # the add is one fp32 add: scores that tie only after rounding tie
    logits = np.array([[1.0, 1.0]], np.float32)
    bias = np.array([0.0, 2.0 ** -24], np.float32)  # fp32: 1 + 2^-24 -> 1 (tie, even)
    sel, _ = orc.route(logits, bias, 1)
    assert sel.tolist() == [[0]]                     # a double add would pick expert 1


@pytest.mark.parametrize("k,E", [(1, 4), (2, 8), (8, 128), (10, 512)])
def test_all_equal_logits(orc, k, E):
    logits = np.full((3, E), 0.25, np.float32)
    sel, w = orc.route(logits, None, k)
    assert np.all(sel == np.arange(k, dtype=np.uint32))
    assert np.all(w == np.float32(1.0 / k))


def test_signed_zero_tie_and_two_expert_closed_form(orc):
    sel, w = orc.route(np.array([[-0.0, 0.0, -1.0]], np.float32), None, 2)
    assert sel.tolist() == [[0, 1]] and w.tolist() == [[0.5, 0.5]]
    for d in [0.1, 1.0, 3.5, 10.0]:
        sel, w = orc.route(np.array([[0.0, d]], np.float32), None, 2)
        assert sel.tolist() == [[1, 0]]
        assert w[0, 0] == np.float32(sp.expit(np.float64(np.float32(d))))


def stable_dispatch(sel, E):
    T, k = sel.shape
    flat = sel.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    row_src = (order // k).astype(np.int32)
    row_experts = flat[order].astype(np.uint32)
    slot_pos = np.empty(T * k, np.int32)
    slot_pos[order] = np.arange(T * k, dtype=np.int32)
    offsets = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]).astype(np.int32)
    return offsets, row_src, slot_pos.reshape(T, k), row_experts


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (64, 128, 8), (300, 512, 10), (1, 4, 4)])
def test_dispatch_matches_stable_argsort(orc, T, E, k):
    rng = np.random.default_rng(T + E)
    sel, _ = orc.route(rng.normal(0, 1, (T, E)).astype(np.float32), None, k)
    got = orc.dispatch_index(sel, E)
    ref = stable_dispatch(sel, E)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)
    off, src, pos, rex = got
    assert off[-1] == T * k
    assert np.all(np.diff(rex.astype(np.int64)) >= 0)
    for e in range(E):                                   # token order inside an expert
        assert np.all(np.diff(src[off[e]:off[e + 1]]) > 0)


def test_copy_rows_are_bit_copies(orc):
    rng = np.random.default_rng(3)
    x = rng.integers(0, 65536, size=(20, 33), dtype=np.uint16)   # arbitrary bf16 bits
    sel, _ = orc.route(rng.normal(0, 1, (20, 6)).astype(np.float32), None, 3)
    _, src, _, _ = orc.dispatch_index(sel, 6)
    values = orc.copy_rows(x, src)
    np.testing.assert_array_equal(values, x[src])


def test_counts(orc):
    rng = np.random.default_rng(5)
    T, E, k = 100, 16, 4
    sel, _ = orc.route(rng.normal(0, 1, (T, E)).astype(np.float32), None, k)
    off, _, _, _ = orc.dispatch_index(sel, E)
    assert orc.counts(off, [0, E]).tolist() == [T * k]
    np.testing.assert_array_equal(orc.counts(off, np.arange(E + 1)),
                                  np.bincount(sel.reshape(-1), minlength=E))
    c = orc.counts(off, [0, 4, 4, 10, 16])
    h = np.bincount(sel.reshape(-1), minlength=E)
    assert c.tolist() == [h[0:4].sum(), 0, h[4:10].sum(), h[10:16].sum()]
    assert orc.counts(off, [3]).tolist() == []
    for bad in ([0, 17], [4, 2], [-1, 3]):
        with pytest.raises(ValueError):
            orc.counts(off, bad)
