"""Seeded synthetic inputs for one MoE decode FFN layer with a gated shared expert.

This module only draws random numbers and encodes them in the storage formats
the layer consumes (fp32, bf16, 4-bit blocks).  It holds none of the layer's
arithmetic, so both the CPU oracle and the GPU library can be fed from it
without sharing any computation.

Distributions (the pages publish no weights; these stand in for a trained
layer of the same shapes):

* router rows and the shared-gate vector: N(0, 0.02) (standard deviation), fp32;
* expert and shared FFN weights: N(0, 0.02) drawn in fp32 then rounded to
  nearest-even bf16, or 4-bit symmetric blocks: integer q uniform in [-8, 7],
  one fp16 scale per 32-element block drawn U(0.001, 0.01) in fp32 then
  rounded to fp16;
* tokens: i.i.d. N(0, 1), stored as bf16 (or fp32 for the all-fp32 layer);
* the optional input-norm weights: U(0.5, 1.5), fp32.

4-bit block layout ("Q4_B32"): a block is 32 consecutive elements along the
input (reduction) dimension of a weight row.  Element j of a block lives in
byte j // 2 of the block's 16 bytes, even j in the low nibble and odd j in the
high nibble, stored unsigned as u = q + 8.  Scales are a separate fp16 tensor
with one entry per (row, block).

Every matrix is generated expert by expert, each from its own stream
``SeedSequence(seed, spawn_key=(matrix_id, expert))``, so a layer is a
deterministic function of its seed whatever the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

WEIGHT_STD = 0.02
Q4_BLOCK = 32
Q4_SCALE_LO = 0.001
Q4_SCALE_HI = 0.01

# matrix ids used in the per-expert spawn keys (fixed generation order)
_MID_ROUTER, _MID_GATE, _MID_UP, _MID_DOWN = 0, 1, 2, 3
_MID_SH_GATE, _MID_SH_UP, _MID_SH_DOWN, _MID_GVEC, _MID_X = 4, 5, 6, 7, 8
_MID_NORM = 9

# weights of the optional input RMSNorm: U(0.5, 1.5), fp32 (a trained norm's
# per-channel gains sit around one)
NORM_W_LO, NORM_W_HI = 0.5, 1.5


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    x_dtype: str = "bf16"   # "f32" | "bf16"
    w_dtype: str = "bf16"   # "f32" | "bf16" | "q4"

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


# The workloads: a tiny all-fp32 layer the oracle finishes instantly, and the
# decode layer (hidden 2048, 256 experts, top-8, expert and shared inter 512)
# in bf16 and 4-bit-block weight storage at several token counts.
TINY = LayerShape(64, 8, 2, 32, 32, "f32", "f32")
DECODE_BF16 = LayerShape(2048, 256, 8, 512, 512, "bf16", "bf16")
DECODE_Q4 = LayerShape(2048, 256, 8, 512, 512, "bf16", "q4")
# one GPU's share of the decode layer split eight ways inside every expert (each GPU
# holds 64 of the 512 intermediate rows of every expert and of the shared expert;
# the router is replicated): the same kernels at the shard's real shape
DECODE_BF16_TP8 = LayerShape(2048, 256, 8, 64, 64, "bf16", "bf16")

WORKLOADS = {
    # name: (shape, seed, token counts)
    "tiny_fp32": (TINY, 0, (1,)),
    "decode_bf16_t1": (DECODE_BF16, 1, (1,)),
    "decode_bf16_t8": (DECODE_BF16, 2, (8,)),
    "decode_q4_t1_t4": (DECODE_Q4, 3, (1, 4)),
    "decode_q4_t1": (DECODE_Q4, 3, (1,)),
    "decode_bf16_t128": (DECODE_BF16, 4, (128,)),
    # prefill chunks: every expert busy, ~128 and ~512 tokens per expert
    "prefill_bf16_t4096": (DECODE_BF16, 5, (4096,)),
    "prefill_bf16_t16384": (DECODE_BF16, 6, (16384,)),
    # one GPU's shard of the layer split eight ways inside every expert
    "decode_bf16_t1_tp8": (DECODE_BF16_TP8, 7, (1,)),
    "decode_bf16_t8_tp8": (DECODE_BF16_TP8, 9, (8,)),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _stream(seed: int, mid: int, idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(mid, idx))))


def _normal_f32(seed: int, mid: int, n_mats: int, rows: int, cols: int, std: float) -> np.ndarray:
    out = np.empty((n_mats, rows, cols), dtype=np.float32)

    def one(e: int) -> None:
        g = _stream(seed, mid, e)
        out[e] = g.standard_normal((rows, cols), dtype=np.float32)
        if std != 1.0:
            out[e] *= np.float32(std)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(n_mats)))
    return out


def _q4_blocks(seed: int, mid: int, n_mats: int, rows: int, cols: int):
    assert cols % Q4_BLOCK == 0
    packed = np.empty((n_mats, rows, cols // 2), dtype=np.uint8)
    scales = np.empty((n_mats, rows, cols // Q4_BLOCK), dtype=np.float32)

    def one(e: int) -> None:
        g = _stream(seed, mid, e)
        q = g.integers(-8, 8, size=(rows, cols), dtype=np.int8)
        u = (q + 8).astype(np.uint8)
        packed[e] = u[:, 0::2] | (u[:, 1::2] << 4)
        scales[e] = g.uniform(Q4_SCALE_LO, Q4_SCALE_HI, size=(rows, cols // Q4_BLOCK)).astype(np.float32)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(n_mats)))
    return torch.from_numpy(packed), torch.from_numpy(scales).to(torch.float16)


def _ffn_matrix(shape: LayerShape, seed: int, mid: int, n_mats: int, rows: int, cols: int) -> dict:
    """One stack of FFN matrices [n_mats, rows, cols] in the layer's weight storage."""
    if shape.w_dtype == "q4":
        packed, scales = _q4_blocks(seed, mid, n_mats, rows, cols)
        return {"w": packed, "scale": scales}
    w = torch.from_numpy(_normal_f32(seed, mid, n_mats, rows, cols, WEIGHT_STD))
    if shape.w_dtype == "bf16":
        w = w.to(torch.bfloat16)
    elif shape.w_dtype != "f32":
        raise ValueError(f"unknown weight dtype {shape.w_dtype}")
    return {"w": w, "scale": None}


def make_layer(shape: LayerShape, seed: int) -> dict:
    """All weights of one layer as CPU tensors.

    Keys: router [E,H] f32; gate, up [E,I,H]; down [E,H,I]; sh_gate, sh_up
    [I_s,H]; sh_down [H,I_s]; gate_vec [H] f32.  For "q4" storage each FFN
    matrix is uint8 [..., K/2] and a matching "<name>_scale" fp16 [..., K/32]
    holds the block scales (None otherwise).
    """
    H, E, I, Is = shape.hidden, shape.n_experts, shape.inter, shape.shared_inter
    layer = {"shape": shape, "seed": seed}
    layer["router"] = torch.from_numpy(_normal_f32(seed, _MID_ROUTER, 1, E, H, WEIGHT_STD)[0])
    for name, mid, n, r, c in (("gate", _MID_GATE, E, I, H), ("up", _MID_UP, E, I, H),
                               ("down", _MID_DOWN, E, H, I), ("sh_gate", _MID_SH_GATE, 1, Is, H),
                               ("sh_up", _MID_SH_UP, 1, Is, H), ("sh_down", _MID_SH_DOWN, 1, H, Is)):
        m = _ffn_matrix(shape, seed, mid, n, r, c)
        w, s = m["w"], m["scale"]
        if name.startswith("sh_"):
            w = w[0]
            s = None if s is None else s[0]
        layer[name] = w.contiguous()
        layer[name + "_scale"] = None if s is None else s.contiguous()
    layer["gate_vec"] = torch.from_numpy(_normal_f32(seed, _MID_GVEC, 1, 1, H, WEIGHT_STD)[0, 0])
    return layer


def make_norm_weight(shape: LayerShape, seed: int) -> torch.Tensor:
    """[H] fp32 weights of the input RMSNorm, U(0.5, 1.5)."""
    g = _stream(seed, _MID_NORM, 0)
    return torch.from_numpy(g.uniform(NORM_W_LO, NORM_W_HI, shape.hidden).astype(np.float32))


def with_input_block(layer: dict, seed: int, eps: float = 1e-6, norm: bool = True,
                     residual: bool = True) -> dict:
    """A copy of `layer` that also carries the input RMSNorm (norm_w, norm_eps)
    and/or the residual add (the keys the binding and the oracle read)."""
    out = dict(layer)
    if norm:
        w = make_norm_weight(layer["shape"], seed)
        dev = layer["gate_vec"].device
        out["norm_w"] = w.to(dev)
        out["norm_eps"] = float(eps)
    out["residual"] = bool(residual)
    return out


def make_tokens(shape: LayerShape, n_tokens: int, seed: int, stream: int = 0) -> torch.Tensor:
    """[n_tokens, H] i.i.d. N(0,1) tokens in the layer's activation storage."""
    g = _stream(seed, _MID_X, stream)
    x = torch.from_numpy(g.standard_normal((n_tokens, shape.hidden), dtype=np.float32))
    if shape.x_dtype == "bf16":
        x = x.to(torch.bfloat16)
    elif shape.x_dtype != "f32":
        raise ValueError(f"unknown activation dtype {shape.x_dtype}")
    return x.contiguous()


def make_layer_device(shape: LayerShape, seed: int, device) -> dict:
    """Same shapes and distributions as make_layer, drawn on the device.

    Used for the many timing copies of a layer, where only the distribution
    matters; the numbers differ from make_layer's.
    """
    H, E, I, Is = shape.hidden, shape.n_experts, shape.inter, shape.shared_inter
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(*size, std=WEIGHT_STD):
        return torch.randn(*size, generator=g, device=device, dtype=torch.float32).mul_(std)

    def ffn(n, r, c):
        if shape.w_dtype == "q4":
            q = torch.randint(-8, 8, (n, r, c), generator=g, device=device, dtype=torch.int16)
            u = (q + 8).to(torch.uint8)
            packed = (u[..., 0::2] | (u[..., 1::2] << 4)).contiguous()
            sc = torch.rand(n, r, c // Q4_BLOCK, generator=g, device=device)
            sc = sc.mul_(Q4_SCALE_HI - Q4_SCALE_LO).add_(Q4_SCALE_LO).to(torch.float16)
            return packed, sc
        out = torch.empty(n, r, c, device=device,
                          dtype=torch.bfloat16 if shape.w_dtype == "bf16" else torch.float32)
        for e in range(n):  # bounded temporaries
            out[e] = normal(r, c)
        return out, None

    layer = {"shape": shape, "seed": seed, "router": normal(E, H)}
    for name, n, r, c in (("gate", E, I, H), ("up", E, I, H), ("down", E, H, I),
                          ("sh_gate", 1, Is, H), ("sh_up", 1, Is, H), ("sh_down", 1, H, Is)):
        w, s = ffn(n, r, c)
        if name.startswith("sh_"):
            w = w[0]
            s = None if s is None else s[0]
        layer[name] = w.contiguous()
        layer[name + "_scale"] = None if s is None else s.contiguous()
    layer["gate_vec"] = normal(H)
    return layer


def make_tokens_device(shape: LayerShape, n_tokens: int, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(n_tokens, shape.hidden, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if shape.x_dtype == "bf16" else x


def layer_to(layer: dict, device) -> dict:
    """Copy every tensor of a layer to `device` (other keys unchanged)."""
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}
