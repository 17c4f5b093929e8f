"""Seeded synthetic inputs for the routed MoE expert FFN.

This module only draws inputs: it holds none of the method's arithmetic (no
routing, no dequantisation, no projection).  Both the HIP path and the CPU oracle
are fed from it.  Arrays are numpy in storage form: fp32 -> float32, fp16 ->
float16, bf16 -> uint16 bit patterns, AWQ words -> int32, MXFP4 bytes -> uint8.

Recipe (one numpy ``default_rng(seed)`` stream per config, draws in a fixed order):
  * "N(0, s)" values are drawn in float64 and rounded to the storage type
    (bf16 through float32, ties to even);
  * AWQ qweight / qzeros are uniform random 32-bit words, so every 4-bit code and
    zero point is uniform on 0..15;
  * scales are uniform on the stated interval;
  * MXFP4 block bytes are uniform random bytes (every E2M1 code equally likely),
    E8M0 scale bytes uniform in 119..125 (2^-8 .. 2^-2);
  * router logits are float32 N(0,1); the prefill-shaped config adds a per-expert
    bias N(0, 0.5); the many-expert config adds a Zipf(1.1)-ranked bias
    b_e = -1.1 * ln(rank_e), rank_e = 1 + position of e in a seeded permutation.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # tokens
    H: int            # hidden (input features of gate/up, output of down)
    I: int            # intermediate
    E: int            # experts
    k: int            # top_k
    group: int        # AWQ group size (MXFP4: the 32-element block)
    adt: str          # activation storage: "f32" | "bf16"
    sdt: str          # AWQ scale storage: "f32" | "f16" | "bf16"
    fmt: str = "awq"  # "awq" | "mxfp4"
    scale_lo: float = 0.002
    scale_hi: float = 0.01
    router_bias: str = "none"   # "none" | "normal" | "zipf"
    router_bias_std: float = 0.5
    zipf_s: float = 1.1
    awq_bias: bool = False
    clamp: float = 0.0

    @property
    def A(self) -> int:
        return self.T * self.k


# The five workloads the method is measured on.
CONFIGS = {
    "tiny": MoeConfig("tiny", T=16, H=128, I=256, E=8, k=2, group=32, adt="f32", sdt="f16",
                      scale_lo=0.005, scale_hi=0.02),
    "decode": MoeConfig("decode", T=64, H=2048, I=768, E=128, k=8, group=128, adt="bf16",
                        sdt="bf16"),
    "prefill": MoeConfig("prefill", T=4096, H=2048, I=768, E=128, k=8, group=128, adt="bf16",
                         sdt="bf16", router_bias="normal"),
    "many": MoeConfig("many", T=1024, H=2048, I=512, E=512, k=10, group=128, adt="bf16",
                      sdt="f32", router_bias="zipf", awq_bias=True),
    "mxfp4": MoeConfig("mxfp4", T=2048, H=2880, I=2880, E=128, k=4, group=32, adt="bf16",
                       sdt="bf16", fmt="mxfp4", clamp=7.0),
}
CONFIG_ORDER = ["tiny", "decode", "prefill", "many", "mxfp4"]
DEFAULT_SEED = {name: 1000 + i for i, name in enumerate(CONFIG_ORDER)}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, ties to even (input generation only)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def to_storage(a64: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return a64.astype(np.float32)
    if dt == "f16":
        return a64.astype(np.float16)
    if dt == "bf16":
        return f32_to_bf16_bits(a64.astype(np.float32))
    raise ValueError(dt)


def storage_to_f64(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact widening of storage values to float64 (for comparisons)."""
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)


def awq_cube(rng, E, K, N, group, sdt, lo, hi, with_bias=False):
    """One AWQ expert cube: qweight [E,K,N/8], qzeros [E,K/g,N/8], scales [E,K/g,N]."""
    qw = random_words(rng, (E, K, N // 8))
    qz = random_words(rng, (E, K // group, N // 8))
    s = to_storage(rng.uniform(lo, hi, size=(E, K // group, N)), sdt)
    b = None
    if with_bias:
        # bf16 N(0, 0.01) values, held in the scale dtype
        b16 = to_storage(rng.normal(0.0, 0.01, size=(E, N)), "bf16")
        b = to_storage(storage_to_f64(b16, "bf16"), sdt)
    return qw, qz, s, b


def router_inputs(rng, cfg: MoeConfig):
    logits = rng.normal(0.0, 1.0, size=(cfg.T, cfg.E)).astype(np.float32)
    bias: Optional[np.ndarray] = None
    if cfg.router_bias == "normal":
        bias = rng.normal(0.0, cfg.router_bias_std, size=cfg.E).astype(np.float32)
    elif cfg.router_bias == "zipf":
        rank = 1 + rng.permutation(cfg.E)
        bias = (-cfg.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return logits, bias


def make_inputs(cfg: MoeConfig, seed: Optional[int] = None, T: Optional[int] = None) -> dict:
    """All inputs of one forward pass.  ``T`` overrides the token count (same recipe)."""
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    if seed is None:
        seed = DEFAULT_SEED.get(cfg.name, 1234)
    rng = np.random.default_rng(seed)
    p = dict(fmt=cfg.fmt, T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k, group=cfg.group,
             adt=cfg.adt, sdt=cfg.sdt, clamp=cfg.clamp, alpha=1.0, up_offset=0.0, cfg=cfg)
    p["x"] = to_storage(rng.normal(0.0, 1.0, size=(cfg.T, cfg.H)), cfg.adt)
    p["logits"], p["router_bias"] = router_inputs(rng, cfg)
    if cfg.fmt == "awq":
        for nm, (K, N) in (("gate", (cfg.H, cfg.I)), ("up", (cfg.H, cfg.I)),
                           ("down", (cfg.I, cfg.H))):
            qw, qz, s, b = awq_cube(rng, cfg.E, K, N, cfg.group, cfg.sdt, cfg.scale_lo,
                                    cfg.scale_hi, cfg.awq_bias)
            p[nm + "_qw"], p[nm + "_qz"], p[nm + "_s"], p[nm + "_b"] = qw, qz, s, b
    else:
        E, H, I = cfg.E, cfg.H, cfg.I
        p["gu_blocks"] = rng.integers(0, 256, size=(E, 2 * I, H // 32, 16), dtype=np.uint8)
        p["gu_scales"] = rng.integers(119, 126, size=(E, 2 * I, H // 32), dtype=np.uint8)
        p["gu_bias"] = to_storage(rng.normal(0.0, 0.01, size=(E, 2 * I)), "bf16")
        p["dn_blocks"] = rng.integers(0, 256, size=(E, H, I // 32, 16), dtype=np.uint8)
        p["dn_scales"] = rng.integers(119, 126, size=(E, H, I // 32), dtype=np.uint8)
        p["dn_bias"] = to_storage(rng.normal(0.0, 0.01, size=(E, H)), "bf16")
    return p


def weight_bytes(p: dict) -> int:
    """Bytes of all expert weight arrays in an inputs dict."""
    keys = [k for k in p if k.endswith(("_qw", "_qz", "_s", "_b", "_blocks", "_scales", "_bias"))
            and k != "router_bias"]
    return sum(int(p[k].nbytes) for k in keys if isinstance(p[k], np.ndarray))
