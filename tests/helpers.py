"""Plumbing between the synthetic-input tensors and the oracle's numpy arrays.

No arithmetic of the layer lives here: only dtype views and copies.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.oracle import OracleLayer


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp16 tensor -> its uint16 bit patterns."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def stored(t: torch.Tensor | None) -> np.ndarray | None:
    """A stored tensor in the oracle's representation (bit patterns for 16-bit types)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return bits16(t)
    return t.numpy()


def oracle_layer(layer: dict) -> OracleLayer:
    s = layer["shape"]
    return OracleLayer(
        hidden=s.hidden, n_experts=s.n_experts, top_k=s.top_k, inter=s.inter,
        shared_inter=s.shared_inter, x_kind=s.x_dtype, w_kind=s.w_dtype,
        router=stored(layer["router"]), gate=stored(layer["gate"]), up=stored(layer["up"]),
        down=stored(layer["down"]), sh_gate=stored(layer["sh_gate"]), sh_up=stored(layer["sh_up"]),
        sh_down=stored(layer["sh_down"]), gate_vec=stored(layer["gate_vec"]),
        gate_scale=stored(layer["gate_scale"]), up_scale=stored(layer["up_scale"]),
        down_scale=stored(layer["down_scale"]), sh_gate_scale=stored(layer["sh_gate_scale"]),
        sh_up_scale=stored(layer["sh_up_scale"]), sh_down_scale=stored(layer["sh_down_scale"]),
        # the plan takes eps as fp32: the oracle gets that same value
        norm_w=stored(layer.get("norm_w")), norm_eps=float(np.float32(layer.get("norm_eps", 0.0))),
        residual=bool(layer.get("residual", False)))


def oracle_tokens(x: torch.Tensor) -> np.ndarray:
    return stored(x)
