"""Shared helpers for the GPU tests: run the HIP layer through the C ABI, run
the oracle on the same bytes, and compare them under the routing near-tie rule.

Near-tie rule: on the oracle's fp64 logits, sort each token's experts; a gap
below NEAR_TIE between ranks k and k+1 (the selection boundary) flags the
token, which is then left out of the id comparison and checked instead against
an oracle run forced to the GPU's ids; a gap below NEAR_TIE between two
selected ranks only excuses their order.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from moe_decode_ffn_amd import ffn
from tests.helpers import oracle_layer, oracle_tokens

NEAR_TIE = 1e-5
TOL_F32 = 1e-4
TOL_LOWP = 2e-2


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def oracle_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return 1


def tol_for(shape) -> float:
    return TOL_F32 if shape.w_dtype == "f32" else TOL_LOWP


def run_gpu(mf: ffn.MoeFfn, layer_dev: dict, x_dev: torch.Tensor, ws: torch.Tensor | None = None,
            out: torch.Tensor | None = None, stream=None, poison: int | None = None) -> dict:
    """One forward with every debug output; returns CPU tensors."""
    dev = x_dev.device
    T = x_dev.shape[0]
    s = layer_dev["shape"]
    if ws is None:
        ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    if poison is not None:
        ws.fill_(poison)
    if out is None:
        out = torch.full((T, s.hidden), float("nan"), dtype=torch.float32, device=dev)
    dbg = {"ids": torch.full((T, s.top_k), -1, dtype=torch.int32, device=dev),
           "weights": torch.empty(T, s.top_k, dtype=torch.float32, device=dev),
           "logits": torch.empty(T, s.n_experts, dtype=torch.float32, device=dev),
           "gate": torch.empty(T, dtype=torch.float32, device=dev)}
    mf.forward(layer_dev, x_dev, out, ws, stream=stream, dbg=dbg)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in dbg.items()}
    res["out"] = out.cpu()
    return res


def near_tie_flags(logits: np.ndarray, k: int):
    """(boundary_flag[T], order_flag[T, k-1]) from fp64 logits."""
    srt = -np.sort(-logits, axis=1)
    gaps = srt[:, :-1] - srt[:, 1:]
    boundary = gaps[:, k - 1] < NEAR_TIE if logits.shape[1] > k else np.zeros(len(logits), bool)
    order = gaps[:, : k - 1] < NEAR_TIE
    return boundary, order


def compare(orc, layer_cpu: dict, x_cpu: torch.Tensor, got: dict, tol: float, ref: dict | None = None,
            nthreads: int | None = None) -> dict:
    """Asserts the GPU result matches the oracle; returns a small report."""
    L = oracle_layer(layer_cpu)
    xo = oracle_tokens(x_cpu)
    nthreads = nthreads or oracle_threads()
    if ref is None:
        ref = orc.forward(L, xo, nthreads=nthreads)
    k = L.top_k
    gids = got["ids"].numpy()
    boundary, order = near_tie_flags(ref["logits"], k)
    ok_tok = ~boundary
    # routing ids: bit-exact except order among near-tied selected ranks
    for t in np.nonzero(ok_tok)[0]:
        if order[t].any():
            assert set(gids[t].tolist()) == set(ref["ids"][t].tolist()), f"token {t}: expert set"
        else:
            assert np.array_equal(gids[t], ref["ids"][t]), f"token {t}: ids {gids[t]} vs {ref['ids'][t]}"
    # routing weights, sums, gate, logits
    gw = got["weights"].double().numpy()
    assert np.all(np.abs(gw.sum(axis=1) - 1.0) <= 1e-5), "renormalised weights must sum to 1"
    gl = got["logits"].double().numpy()
    assert np.max(np.abs(gl - ref["logits"])) <= 1e-4, "router logits"
    assert np.max(np.abs(got["gate"].double().numpy() - ref["gate"])) <= 1e-5, "shared gate"
    for t in np.nonzero(ok_tok & ~order.any(axis=1))[0]:
        assert np.max(np.abs(gw[t] - ref["weights"][t])) <= 1e-5, f"token {t}: weights"
    # output within tolerance of the oracle (relative to the run's max |ref|).  With the
    # residual add the layer's own part, out - x, is judged (x would otherwise set the
    # scale); the last fp32 add may round by half an ulp of out on top of that part's error
    out = got["out"].double().numpy()
    assert np.all(np.isfinite(out)), "non-finite output"
    x0 = x_cpu.double().numpy() if L.residual else np.zeros_like(out)
    slack = np.abs(out) * 2.0**-24 if L.residual else np.zeros_like(out)

    def dev(a, b, rows):
        return float(np.max(np.abs((a[rows] - x0[rows]) - (b[rows] - x0[rows])) - slack[rows]))

    part = ref["out"] - x0
    scale = float(np.max(np.abs(part[ok_tok]))) if ok_tok.any() else 1.0
    err = max(0.0, dev(out, ref["out"], ok_tok)) if ok_tok.any() else 0.0
    assert err <= tol * scale, f"max|d| {err:.3e} > {tol} * {scale:.3e}"
    # boundary-flagged tokens: against the oracle forced to the GPU's ids
    if boundary.any():
        forced = orc.forward(L, xo, nthreads=nthreads, forced_ids=np.where(boundary[:, None], gids, ref["ids"]))
        for t in np.nonzero(boundary)[0]:
            e = dev(out, forced["out"], [t])
            fs = float(np.max(np.abs(forced["out"][t] - x0[t])))
            assert e <= tol * max(scale, fs), f"flagged token {t}"
    return {"rel_err": err / scale if scale else 0.0, "flagged": int(boundary.sum()),
            "order_flagged": int(order.any(axis=1).sum()), "unique_experts": int(len(np.unique(gids)))}
