"""Move a seeded synthetic inputs dict (numpy storage arrays) onto the GPU.

Marshalling only: bit patterns are reinterpreted, never converted.
"""
from __future__ import annotations

import numpy as np
import torch

from . import moeq


def tensor(a: np.ndarray, dt: str, device) -> torch.Tensor:
    """Storage array -> torch tensor with the same bits (bf16 arrives as uint16)."""
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dt == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, np.float16)).to(device)
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    if dt == "i32":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)
    if dt == "u8":
        return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(device)
    raise ValueError(dt)


def to_host(t: torch.Tensor, dt: str) -> np.ndarray:
    """Device tensor -> storage array (bf16 -> uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(p: dict, device="cuda") -> dict:
    """Device copies of x, logits, router bias and the expert payloads."""
    d = dict(x=tensor(p["x"], p["adt"], device), logits=tensor(p["logits"], "f32", device),
             router_bias=None if p["router_bias"] is None
             else tensor(p["router_bias"], "f32", device))
    if p["fmt"] == "awq":
        for nm in ("gate", "up", "down"):
            b = p[nm + "_b"]
            d[nm] = moeq.AwqExperts(tensor(p[nm + "_qw"], "i32", device),
                                    tensor(p[nm + "_qz"], "i32", device),
                                    tensor(p[nm + "_s"], p["sdt"], device), p["group"],
                                    None if b is None else tensor(b, p["sdt"], device))
        d["up_arg"] = d["up"]
    else:
        d["gate"] = moeq.Mxfp4Bank(tensor(p["gu_blocks"], "u8", device),
                                   tensor(p["gu_scales"], "u8", device),
                                   tensor(p["gu_bias"], "bf16", device), True)
        d["down"] = moeq.Mxfp4Bank(tensor(p["dn_blocks"], "u8", device),
                                   tensor(p["dn_scales"], "u8", device),
                                   tensor(p["dn_bias"], "bf16", device), False)
        d["up_arg"] = None
    return d
