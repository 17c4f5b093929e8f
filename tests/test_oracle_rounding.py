"""Oracle storage-rounding helpers against hand-derived bit patterns and numpy."""
import numpy as np
import pytest

from conftest import read_golden


def test_golden_storage_rounding(orc):
    for dt, expr, bits in read_golden("storage_rounding.txt"):
        v = eval(expr, {"__builtins__": {}})  # fixture expressions: numbers and ** only
        got = orc.round_f16_bits(v) if dt == "f16" else orc.round_bf16_bits(v)
        assert got == int(bits, 16), (dt, expr, hex(got), bits)


def test_f16_matches_numpy_cast():
    """numpy's float64 -> float16 cast rounds once, ties to even."""
    import oracle
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 1e-5, 2000),
                           rng.normal(0, 3e4, 2000),
                           # exact ties at several binades
                           (np.arange(1, 200) + 0.5) * 2.0 ** -10,
                           (np.arange(1, 200) + 0.5) * 2.0 ** -24])
    for v in vals:
        assert oracle.round_f16_bits(v) == int(np.float16(v).view(np.uint16)), v


def test_bf16_matches_torch_when_fp32_exact():
    """For values exact in fp32, torch's fp32 -> bf16 rounding is the single rounding."""
    import torch
    import oracle
    rng = np.random.default_rng(8)
    vals = rng.normal(0, 1, 5000).astype(np.float32).astype(np.float64)
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    for v, r in zip(vals, ref.astype(np.uint16)):
        assert oracle.round_bf16_bits(v) == int(r), v


def test_values_roundtrip(orc):
    for bits in [0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC000, 0x8001]:
        assert orc.round_f16_bits(orc.f16_value(bits)) == bits
        assert np.float16(orc.f16_value(bits)).view(np.uint16) == bits
    for bits in [0x0001, 0x3F80, 0x3F81, 0x7F7F, 0xBF81, 0x0080]:
        assert orc.round_bf16_bits(orc.bf16_value(bits)) == bits
