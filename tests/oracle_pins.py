"""Pins that tie the CPU oracle to things other than itself.

Each ``pin_*`` takes a loaded ``Oracle`` and raises AssertionError when the
oracle disagrees with:

* a library routine of the same quantity (torch / numpy conversions, fp64
  matmul, softmax, topk, linear/silu);
* a special case that collapses the layer to a textbook computation
  (one expert; every expert selected; identical experts; zeroed branches);
* hand-derived fixtures under tests/golden/ (closed-form tiny layers and
  4-bit block decodes);
* invariants (renormalised weights sum to one, power-of-two homogeneity,
  expert-permutation equivariance);
* the independent numpy brute-force twin, which evaluates every expert.

The same functions run against deliberately broken builds of the oracle in
test_oracle_mutants.py, which checks that each planted mistake trips at least
one pin.  ``python -m tests.oracle_pins <library.so>`` prints a JSON verdict
per pin (used by that test to isolate broken builds in a subprocess).
"""
from __future__ import annotations

import dataclasses
import json
import os
import sys

import numpy as np
import torch
import torch.nn.functional as F

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from moe_decode_ffn_amd import synth  # noqa: E402
from oracle.oracle import OracleLayer, brute_force, np_bf16, np_decode, np_f16  # noqa: E402
from tests.helpers import oracle_layer, oracle_tokens  # noqa: E402

GOLDEN = os.path.join(HERE, "golden")


def _layer(shape, seed, n_tokens=3):
    lay = synth.make_layer(shape, seed)
    x = synth.make_tokens(shape, n_tokens, seed)
    return oracle_layer(lay), oracle_tokens(x)


def _x64(L: OracleLayer, x):
    return torch.from_numpy(x.astype(np.float64) if L.x_kind == "f32" else np_bf16(x))


def _w64(L: OracleLayer, name):
    return torch.from_numpy(np_decode(getattr(L, name), getattr(L, name + "_scale"), L.w_kind))


def _torch_ffn(x, g, u, d):
    """Plain SwiGLU FFN with torch fp64 ops: d(silu(g x) * (u x))."""
    return F.linear(F.silu(F.linear(x, g)) * F.linear(x, u), d)


def _close(a, b, rtol=1e-12, atol=1e-13, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= atol + rtol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


SMALL = synth.LayerShape(64, 8, 2, 32, 32, "f32", "f32")
SMALL_BF16 = synth.LayerShape(96, 12, 3, 64, 32, "bf16", "bf16")
SMALL_Q4 = synth.LayerShape(128, 10, 3, 64, 96, "bf16", "q4")


# ---------------------------------------------------------------- decoders

def pin_bf16_decoder_matches_torch(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_matrix(bits.reshape(1, -1), None, "bf16")[0]
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "bf16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "bf16 decode differs from torch"
    assert np.array_equal(np_bf16(bits)[~nan], ref[~nan]), "numpy twin bf16 decode"


def pin_f16_decoder_matches_numpy(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    got = np.array([orc.f16_value(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), nan), "fp16 NaN patterns"
    assert np.array_equal(got[~nan], ref[~nan]), "fp16 decode differs from numpy"
    assert np.array_equal(np_f16(bits)[~nan], ref[~nan]), "numpy twin fp16 decode"


def pin_q4_golden_decode(orc):
    g = json.load(open(os.path.join(GOLDEN, "q4_block_decode.json")))
    cols = g["cols"]
    for row in g["rows"]:
        packed = np.frombuffer(bytes.fromhex("".join(row["bytes_hex"])), dtype=np.uint8)
        scales = np.array([int(h, 16) for h in row["scales_hex"]], dtype=np.uint16)
        want = []
        for run in row["values_rle"]:
            want += list(run["seq"]) * run["repeat"]
        want = np.array(want, dtype=np.float64)
        assert want.size == cols and packed.size == cols // 2
        got = orc.decode_matrix(packed.reshape(1, -1), scales.reshape(1, -1), "q4")[0]
        assert np.array_equal(got, want), "q4 decode differs from the hand-decoded fixture"
        assert np.array_equal(np_decode(packed.reshape(1, -1), scales.reshape(1, -1), "q4")[0], want)


# ---------------------------------------------------------------- closed forms

def _golden_layer(case):
    f = lambda k: np.array(case[k], dtype=np.float32)  # noqa: E731
    E, I, H, Is = case["n_experts"], case["inter"], case["hidden"], case["shared_inter"]
    return OracleLayer(hidden=H, n_experts=E, top_k=case["top_k"], inter=I, shared_inter=Is,
                       x_kind="f32", w_kind="f32", router=f("router"), gate=f("gate"),
                       up=f("up"), down=f("down"), sh_gate=f("sh_gate"), sh_up=f("sh_up"),
                       sh_down=f("sh_down"), gate_vec=f("gate_vec")), f("x")


def pin_golden_closed_form_layers(orc):
    g = json.load(open(os.path.join(GOLDEN, "closed_form_layers.json")))
    for case in g["cases"]:
        L, x = _golden_layer(case)
        r = orc.forward(L, x)
        name = case["name"]
        assert np.array_equal(r["ids"], np.array(case["expect_ids"])), f"{name}: ids {r['ids']}"
        assert np.array_equal(r["weights"], np.array(case["expect_weights"])), f"{name}: weights"
        tol = case["abs_tol"]
        assert np.max(np.abs(r["gate"] - np.array(case["expect_gate"]))) <= max(tol, 0.0), f"{name}: gate"
        err = np.max(np.abs(r["out"] - np.array(case["expect_out"])))
        assert err <= tol, f"{name}: out {r['out']} vs {case['expect_out']}"


def pin_router_logits_are_a_matmul(orc):
    for shape, seed in ((SMALL, 11), (SMALL_BF16, 12)):
        L, x = _layer(shape, seed)
        r = orc.forward(L, x)
        ref = (_x64(L, x) @ torch.from_numpy(L.router.astype(np.float64)).T).numpy()
        _close(r["logits"], ref, what="logits vs fp64 matmul")


def pin_topk_matches_torch_topk(orc):
    for shape, seed in ((SMALL, 21), (SMALL_BF16, 22), (SMALL_Q4, 23)):
        L, x = _layer(shape, seed, n_tokens=5)
        r = orc.forward(L, x)
        vals, idx = torch.topk(torch.from_numpy(r["logits"]), L.top_k, dim=1, sorted=True)
        # the drawn logits have no exact ties, so torch's order is the unique rank order
        assert np.array_equal(r["ids"], idx.numpy().astype(np.int32)), "top-k ids vs torch.topk"


def pin_renormalised_weights_closed_form(orc):
    for shape, seed in ((SMALL, 31), (SMALL_Q4, 32)):
        L, x = _layer(shape, seed, n_tokens=4)
        r = orc.forward(L, x)
        lsel = np.take_along_axis(r["logits"], r["ids"].astype(np.int64), axis=1)
        ref = torch.softmax(torch.from_numpy(lsel), dim=1).numpy()
        _close(r["weights"], ref, what="renormalised top-k weights vs softmax of selected logits")
        _close(r["weights"].sum(axis=1), np.ones(x.shape[0]), what="sum of weights")


def pin_shared_gate_is_sigmoid(orc):
    L, x = _layer(SMALL_BF16, 41)
    r = orc.forward(L, x)
    ref = torch.sigmoid(_x64(L, x) @ torch.from_numpy(L.gate_vec.astype(np.float64))).numpy()
    _close(r["gate"], ref, what="shared gate vs torch.sigmoid")


def pin_single_expert_is_plain_swiglu(orc):
    # E = k = 1: the routed branch is one SwiGLU FFN with weight 1
    for shape, seed in ((synth.LayerShape(64, 1, 1, 48, 32, "f32", "f32"), 51),
                        (synth.LayerShape(96, 1, 1, 64, 32, "bf16", "q4"), 52)):
        L, x = _layer(shape, seed)
        r = orc.forward(L, x)
        X = _x64(L, x)
        routed = _torch_ffn(X, _w64(L, "gate")[0], _w64(L, "up")[0], _w64(L, "down")[0])
        S = _torch_ffn(X, _w64(L, "sh_gate"), _w64(L, "sh_up"), _w64(L, "sh_down"))
        s = torch.sigmoid(X @ torch.from_numpy(L.gate_vec.astype(np.float64)))
        _close(r["routed"], routed.numpy(), what="E=k=1 routed vs torch SwiGLU")
        _close(r["shared"], S.numpy(), what="shared expert vs torch SwiGLU")
        _close(r["out"], (routed + s[:, None] * S).numpy(), what="E=k=1 output")


def pin_all_experts_selected_is_dense_mixture(orc):
    # k = E: the routed branch is the softmax-weighted mixture of every expert
    shape = synth.LayerShape(64, 6, 6, 32, 32, "f32", "f32")
    L, x = _layer(shape, 61)
    r = orc.forward(L, x)
    X = _x64(L, x)
    p = torch.softmax(X @ torch.from_numpy(L.router.astype(np.float64)).T, dim=1)
    Wg, Wu, Wd = _w64(L, "gate"), _w64(L, "up"), _w64(L, "down")
    routed = sum(p[:, e:e + 1] * _torch_ffn(X, Wg[e], Wu[e], Wd[e]) for e in range(shape.n_experts))
    _close(r["routed"], routed.numpy(), what="k=E dense softmax mixture")


def pin_identical_experts_collapse(orc):
    # every expert the same: any selection gives that expert's FFN (weights sum to 1)
    shape = synth.LayerShape(64, 8, 3, 32, 32, "bf16", "bf16")
    L, x = _layer(shape, 71)
    for name in ("gate", "up", "down"):
        w = getattr(L, name)
        setattr(L, name, np.ascontiguousarray(np.broadcast_to(w[2:3], w.shape)))
    r = orc.forward(L, x)
    X = _x64(L, x)
    ffn = _torch_ffn(X, _w64(L, "gate")[0], _w64(L, "up")[0], _w64(L, "down")[0])
    _close(r["routed"], ffn.numpy(), what="identical experts")


def pin_zeroed_branches(orc):
    L, x = _layer(SMALL_BF16, 81)
    base = orc.forward(L, x)
    # gate vector 0 -> s = 1/2 exactly, out = routed + S/2
    L.gate_vec = np.zeros_like(L.gate_vec)
    r = orc.forward(L, x)
    assert np.all(r["gate"] == 0.5), "zero gate vector must give s = 1/2"
    assert np.array_equal(r["out"], r["routed"] + 0.5 * r["shared"]), "s = 1/2 join"
    # shared down zero -> out = routed exactly
    L2, _ = _layer(SMALL_BF16, 81)
    L2.sh_down = np.zeros_like(L2.sh_down)
    r2 = orc.forward(L2, x)
    assert np.array_equal(r2["out"], base["routed"]), "zero shared expert leaves the routed output"
    # routed down zero -> out = s * S
    L3, _ = _layer(SMALL_BF16, 81)
    L3.down = np.zeros_like(L3.down)
    r3 = orc.forward(L3, x)
    assert np.array_equal(r3["out"], base["gate"][:, None] * base["shared"]), "zero routed experts"


def pin_brute_force_twin_agrees(orc):
    for shape, seed, T in ((synth.TINY, 0, 1), (SMALL, 91, 4), (SMALL_BF16, 92, 3),
                           (SMALL_Q4, 93, 2)):
        L, x = _layer(shape, seed, n_tokens=T)
        r = orc.forward(L, x)
        b = brute_force(L, x)
        assert np.array_equal(r["ids"], b["ids"]), f"{shape}: ids vs brute force"
        _close(r["weights"], b["weights"], what="weights vs brute force")
        _close(r["logits"], b["logits"], what="logits vs brute force")
        _close(r["gate"], b["gate"], what="gate vs brute force")
        _close(r["shared"], b["shared"], what="shared vs brute force")
        _close(r["out"], b["out"], what="out vs brute force")
        # the identity out = sum_j w_j E_{ids_j}(x) + s S(x), from the all-expert table
        Y = b["all_experts"]
        for t in range(T):
            mix = sum(r["weights"][t, j] * Y[t, r["ids"][t, j]] for j in range(shape.top_k))
            _close(r["out"][t], mix + r["gate"][t] * b["shared"][t], what="identity")


def pin_tiny_layer_best_pair(orc):
    # E = 8, k = 2 on the tiny layer: among all 28 pairs, the oracle's pair has the two
    # largest logits, and its output equals that pair's renormalised mixture
    L, x = _layer(synth.TINY, 0, n_tokens=1)
    r = orc.forward(L, x)
    b = brute_force(L, x)
    lg = b["logits"][0]
    pairs = [(a, c) for a in range(8) for c in range(a + 1, 8)]
    best = max(pairs, key=lambda pr: lg[pr[0]] + lg[pr[1]])
    assert set(r["ids"][0].tolist()) == set(best), "top-2 set is the best pair"
    a, c = sorted(best, key=lambda e: (-lg[e], e))
    wa = 1.0 / (1.0 + np.exp(lg[c] - lg[a]))
    mix = wa * b["all_experts"][0, a] + (1.0 - wa) * b["all_experts"][0, c]
    _close(r["routed"][0], mix, what="pair mixture")


def pin_power_of_two_homogeneity(orc):
    L, x = _layer(SMALL_BF16, 101)
    base = orc.forward(L, x)
    # bf16 * 2 is exact: doubling every down matrix doubles routed and shared exactly
    two = np.uint16(1 << 7)  # add 1 to the bf16 exponent field
    L.down = np.where((L.down & 0x7F80) != 0, L.down + two, L.down).astype(np.uint16)
    L.sh_down = np.where((L.sh_down & 0x7F80) != 0, L.sh_down + two, L.sh_down).astype(np.uint16)
    r = orc.forward(L, x)
    assert np.array_equal(r["routed"], 2.0 * base["routed"]), "routed homogeneity"
    assert np.array_equal(r["shared"], 2.0 * base["shared"]), "shared homogeneity"


def pin_q4_equals_dequantised_f32(orc):
    Lq, x = _layer(SMALL_Q4, 111)
    rq = orc.forward(Lq, x)
    deq = {n: np_decode(getattr(Lq, n), getattr(Lq, n + "_scale"), "q4").astype(np.float32)
           for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")}
    Lf = OracleLayer(hidden=Lq.hidden, n_experts=Lq.n_experts, top_k=Lq.top_k, inter=Lq.inter,
                     shared_inter=Lq.shared_inter, x_kind=Lq.x_kind, w_kind="f32",
                     router=Lq.router, gate_vec=Lq.gate_vec, **deq)
    rf = orc.forward(Lf, x)
    # scale (11 significant bits) times q (4 bits) is exact in fp32, so both paths see
    # identical values in identical order
    assert np.array_equal(rq["out"], rf["out"]), "4-bit path vs dequantised fp32 path"


def pin_expert_permutation_equivariance(orc):
    L, x = _layer(SMALL_Q4, 121, n_tokens=4)
    r = orc.forward(L, x)
    perm = np.random.default_rng(5).permutation(L.n_experts)
    P = dataclasses.replace(L)
    P.router = L.router[perm]
    for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale"):
        setattr(P, n, np.ascontiguousarray(getattr(L, n)[perm]))
    rp = orc.forward(P, x)
    # expert i of the permuted layer is expert perm[i] of the original
    assert np.array_equal(perm[rp["ids"]], r["ids"]), "permuted ids"
    _close(rp["out"], r["out"], what="permuted experts")


def pin_forced_ids(orc):
    L, x = _layer(SMALL, 131, n_tokens=3)
    r = orc.forward(L, x)
    same = orc.forward(L, x, forced_ids=r["ids"])
    assert np.array_equal(same["out"], r["out"]), "forcing the natural ids changes nothing"
    b = brute_force(L, x)
    forced = np.array([[5, 1], [0, 7], [3, 2]], dtype=np.int32)
    f = orc.forward(L, x, forced_ids=forced)
    for t in range(3):
        lsel = b["logits"][t, forced[t]]
        w = np.exp(lsel - lsel.max())
        w /= w.sum()
        mix = sum(w[j] * b["all_experts"][t, forced[t, j]] for j in range(2))
        _close(f["out"][t], mix + b["gate"][t] * b["shared"][t], what="forced ids")


# ------------------------------------------------- input norm and residual

def _with_block(L: OracleLayer, seed: int, eps: float, residual: bool = True) -> OracleLayer:
    w = np.random.default_rng(seed).uniform(0.5, 1.5, L.hidden).astype(np.float32)
    return dataclasses.replace(L, norm_w=w, norm_eps=eps, residual=residual)


def pin_block_matches_torch_rms_norm(orc):
    # E = k = 1: out = x0 + SwiGLU(rms_norm(x0) * w) + s(.) * S(.), all from torch routines; the
    # tokens are scaled down so that eps is not negligible against their mean square
    for shape, seed, scale in ((synth.LayerShape(64, 1, 1, 48, 32, "f32", "f32"), 151, 0.05),
                               (synth.LayerShape(96, 1, 1, 64, 32, "f32", "q4"), 152, 1.0)):
        L0, x = _layer(shape, seed)
        x = (x * np.float32(scale)).astype(np.float32)
        L = _with_block(L0, seed, eps=1e-3)
        r = orc.forward(L, x)
        X0 = _x64(L, x)
        X = F.rms_norm(X0, (L.hidden,), weight=torch.from_numpy(L.norm_w.astype(np.float64)),
                       eps=L.norm_eps)
        routed = _torch_ffn(X, _w64(L, "gate")[0], _w64(L, "up")[0], _w64(L, "down")[0])
        S = _torch_ffn(X, _w64(L, "sh_gate"), _w64(L, "sh_up"), _w64(L, "sh_down"))
        s = torch.sigmoid(X @ torch.from_numpy(L.gate_vec.astype(np.float64)))
        _close(r["logits"], (X @ torch.from_numpy(L.router.astype(np.float64)).T).numpy(),
               what="logits of the normalised input")
        _close(r["out"], (X0 + (routed + s[:, None] * S)).numpy(), what="norm + layer + residual")
        plain = orc.forward(dataclasses.replace(L, residual=False), x)
        _close(plain["out"], (routed + s[:, None] * S).numpy(), what="norm without residual")


def pin_norm_scale_invariance(orc):
    # eps = 0: RMSNorm removes any positive scale of the input exactly (up to fp64 rounding)
    L0, x = _layer(SMALL, 161)
    L = _with_block(L0, 161, eps=0.0, residual=False)
    a = orc.forward(L, x)
    b = orc.forward(L, (x * np.float32(4.0)).astype(np.float32))
    _close(b["out"], a["out"], rtol=1e-12, what="norm(4 x) = norm(x)")
    assert np.array_equal(a["ids"], b["ids"]), "scaled input must route the same"


def pin_residual_around_a_zero_layer(orc):
    # every FFN weight zero: the layer output is 0 and the block returns its input exactly
    L0, x = _layer(SMALL_BF16, 171)
    L = _with_block(L0, 171, eps=1e-6)
    for name in ("down", "sh_down"):
        setattr(L, name, np.zeros_like(getattr(L, name)))
    r = orc.forward(L, x)
    assert np.array_equal(r["out"], _x64(L, x).numpy()), "zero layer: out = x0"


def pin_brute_force_twin_with_block(orc):
    for shape, seed, T in ((SMALL, 181, 3), (SMALL_BF16, 182, 2), (SMALL_Q4, 183, 2)):
        L0, x = _layer(shape, seed, T)
        L = _with_block(L0, seed, eps=1e-5)
        r = orc.forward(L, x)
        b = brute_force(L, x)
        assert np.array_equal(r["ids"], b["ids"]), "ids with input norm"
        _close(r["out"], b["out"], rtol=1e-11, what="C oracle vs numpy twin, norm + residual")


PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}


def run_all(orc) -> dict:
    verdict = {}
    for name, fn in PINS.items():
        try:
            fn(orc)
            verdict[name] = "pass"
        except AssertionError as e:
            verdict[name] = f"fail: {e}"[:300]
        except Exception as e:  # a broken build may also raise
            verdict[name] = f"error: {type(e).__name__}: {e}"[:300]
    return verdict


if __name__ == "__main__":
    from oracle.oracle import Oracle
    print(json.dumps(run_all(Oracle(sys.argv[1]))))
