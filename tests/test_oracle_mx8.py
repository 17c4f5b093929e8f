"""Oracle of the MXFP8-activation variant of the MXFP4 bank (block-scaled MFMA path):
OCP MX E4M3 element values, the MX quantization of 32-element blocks, and the
projection of quantized rows.

Pins: the E4M3 code table of the OCP MX format (tests/golden/e4m3.txt); blocks
built as 2^E times E4M3 values come back as exactly those codes and scale 127 + E;
round-to-nearest-even at the midpoints; saturation to 448; zero blocks; every
element is the nearest representable value by a brute-force search over all
codes written with numpy; the projection equals a numpy float64 product of the
dequantised rows and the dense bank.
"""
import numpy as np
import pytest

from conftest import read_golden
from quantized_moe_expert_router_amd.synth import to_storage


def e4m3_table(orc):
    return np.array([orc.e4m3_value(c) for c in range(256)])


def test_e4m3_golden(orc):
    for code, val in read_golden("e4m3.txt"):
        got = orc.e4m3_value(int(code, 16))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-")


def test_quantize_exact_blocks_round_trip(orc):
    rng = np.random.default_rng(91)
    tab = e4m3_table(orc)
    finite = [c for c in range(256) if np.isfinite(tab[c])]
    rows, K = 5, 128
    codes = rng.choice(finite, size=(rows, K)).astype(np.uint8)
    E = rng.integers(-20, 20, size=(rows, K // 32))
    # every block's largest magnitude has exponent 8 (256..448): its shared exponent is E
    codes[:, ::32] = rng.choice([0x78, 0x7A, 0x7E, 0xF8, 0xFC], size=(rows, K // 32))
    x = tab[codes] * np.repeat(2.0 ** E, 32, axis=1)
    q, s = orc.mxfp8_quantize(to_storage(x, "f32"), "f32")
    np.testing.assert_array_equal(s, (127 + E).astype(np.uint8))
    np.testing.assert_array_equal(tab[q], tab[codes])     # -0 and +0 compare equal as values


def test_quantize_rounding_saturation_and_zero(orc):
    x = np.zeros((2, 64))
    x[0, :6] = [256.0, 1.0625, 1.1875, -1e-9, 300.0, 0.0]   # shared exponent 0
    x[0, 32] = 500.0 * 2 ** -4                               # block 2: amax 31.25 -> 2^(4-8)
    x[0, 33] = 31.0
    q, s = orc.mxfp8_quantize(to_storage(x, "f32"), "f32")
    assert list(q[0, :6]) == [0x78, 0x38, 0x3A, 0x80, 0x79, 0x00]   # ties to even, signed zero
    assert s[0, 0] == 127 and s[0, 1] == 127 - 4
    # 31.25 / 2^-4 = 500 and 31 / 2^-4 = 496 both exceed 448: saturated
    assert q[0, 32] == 0x7E and q[0, 33] == 0x7E
    assert s[1, 0] == 0 and s[1, 1] == 0 and not q[1].any()         # zero blocks


def test_quantize_is_nearest_code(orc):
    rng = np.random.default_rng(92)
    x = rng.normal(0, 1, (8, 256)) * np.repeat(10.0 ** rng.uniform(-4, 4, (8, 8)), 32, axis=1)
    x = x.astype(np.float32)
    q, s = orc.mxfp8_quantize(x, "f32")
    tab = e4m3_table(orc)
    pos = np.array([tab[c] for c in range(0x7F)])                   # finite non-negative codes
    v = x.astype(np.float64) / np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[..., None] - pos)
    best = np.min(d, axis=-1)
    assert np.all(np.abs(np.abs(tab[q]) - a) == best)
    assert np.all(np.abs(v) / 448.0 < 512.0 / 448.0)                # scale puts the max in range


def test_mx8_project_against_numpy(orc):
    rng = np.random.default_rng(93)
    E, R, C, A = 3, 24, 96, 20
    blocks = rng.integers(0, 256, size=(E, R, C // 32, 16), dtype=np.uint8)
    scales = rng.integers(119, 126, size=(E, R, C // 32), dtype=np.uint8)
    bias = to_storage(rng.normal(0, 0.01, size=(E, R)), "bf16")
    x = to_storage(rng.normal(0, 1, (A, C)), "bf16")
    rex = rng.integers(0, E, size=A).astype(np.uint32)
    q, s = orc.mxfp8_quantize(x, "bf16")
    out = orc.mx8_project(q, s, rex, blocks, scales, bias, "f32").astype(np.float64)
    tab = e4m3_table(orc)
    xv = tab[q] * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    W = orc.mxfp4_dequant(blocks, scales)
    bv = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.stack([xv[p] @ W[rex[p]].T + bv[rex[p]] for p in range(A)])
    np.testing.assert_allclose(out, ref, rtol=2 ** -23, atol=1e-30)
