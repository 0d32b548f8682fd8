"""GPU parity: the HIP layer, called through the C ABI, against the CPU oracle.

Small layers span several workgroup tiles, token passes, router token tiles
and partially covered 16-byte chunk slots; the decode layer (hidden 2048,
256 experts, top-8, inter 512) runs at its real size for batch 1, 8, 128 in
bf16 and batch 1, 4 in 4-bit blocks.  Every shared-expert mode (aux stream,
sequential, fused) must match the oracle and each other bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_decode_ffn_amd import ffn, synth
from tests.gpu_common import TOL_LOWP, compare, device, oracle_threads, run_gpu, tol_for
from tests.helpers import oracle_layer, oracle_tokens

pytestmark = pytest.mark.gpu

MODES = {"aux": ffn.SHARED_AUX, "seq": ffn.SHARED_SEQ, "fused": ffn.SHARED_FUSED}

SMALL = {
    # name: (shape, seed, token counts)
    "tiny_fp32": (synth.TINY, 0, (1, 3)),
    "bf16_ragged_chunks": (synth.LayerShape(160, 12, 3, 96, 64, "bf16", "bf16"), 5, (1, 5, 17)),
    "q4_ragged": (synth.LayerShape(192, 10, 3, 96, 160, "bf16", "q4"), 6, (1, 4, 9)),
    "fp32_two_slots": (synth.LayerShape(288, 20, 4, 64, 96, "f32", "f32"), 7, (2, 11)),
    "bf16_big_buckets": (synth.LayerShape(96, 4, 2, 64, 32, "bf16", "bf16"), 8, (40,)),
    "bf16_k_equals_e": (synth.LayerShape(64, 4, 4, 32, 32, "bf16", "bf16"), 9, (3,)),
    "bf16_one_expert": (synth.LayerShape(96, 1, 1, 64, 32, "bf16", "bf16"), 10, (2,)),
    "q4_wide": (synth.LayerShape(1024, 16, 4, 256, 128, "bf16", "q4"), 11, (1, 6)),
    # top-16: 48 pairs (one-wave sort), 96 and 192 pairs in the gate/up workgroups
    # (workgroup bucketing)
    "bf16_top16": (synth.LayerShape(128, 24, 16, 64, 32, "bf16", "bf16"), 12, (3, 6, 12)),
    # 512 experts: 2 tokens route in the gate/up workgroups; 12 tokens' logits rows exceed
    # what their prologue holds, so the routing launch of its own ranks them
    "bf16_512_experts": (synth.LayerShape(128, 512, 8, 64, 32, "bf16", "bf16"), 13, (2, 12)),
    # 1 KiB rows (64-lane row mapping): 1 token takes the gate/up jobs of one row per
    # wave, 2 to 4 tokens those of two rows per wave
    "bf16_kib_rows": (synth.LayerShape(512, 16, 4, 64, 32, "bf16", "bf16"), 14, (1, 2, 3, 4)),
}


# grouped-GEMM regime (bf16, sizes multiples of 128), forced for every batch:
# buckets of more than 16 tokens (several passes), shared-expert passes of
# 16/32/64 tokens with a ragged last pass, several row tiles per expert
SMALL_GEMM = {
    "gemm_basic": (synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16"), 20, (1, 5, 17)),
    "gemm_big_buckets": (synth.LayerShape(128, 2, 1, 128, 128, "bf16", "bf16"), 21, (40, 100)),
    "gemm_many_tiles": (synth.LayerShape(512, 8, 2, 384, 640, "bf16", "bf16"), 22, (33,)),
    "gemm_k_equals_e": (synth.LayerShape(128, 4, 4, 128, 128, "bf16", "bf16"), 23, (3, 70)),
}


def _plan(shape, max_tokens, mode, extra=0):
    return ffn.MoeFfn.for_shape(shape, max_tokens=max_tokens, flags=MODES[mode] | extra)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layers_all_modes(orc, name):
    dev = device()
    shape, seed, counts = SMALL[name]
    layer = synth.make_layer(shape, seed)
    dl = synth.layer_to(layer, dev)
    plans = {m: _plan(shape, max(counts), m) for m in MODES}
    for T in counts:
        x = synth.make_tokens(shape, T, seed, stream=T)
        ref = orc.forward(oracle_layer(layer), oracle_tokens(x))
        outs = {}
        for m, mf in plans.items():
            print(f"[small] {name} T={T} mode={m}", flush=True)
            got = run_gpu(mf, dl, x.to(dev))
            compare(orc, layer, x, got, tol_for(shape), ref=ref)
            outs[m] = got["out"]
        assert torch.equal(outs["aux"], outs["seq"]), "aux vs sequential must be bit-identical"
        assert torch.equal(outs["aux"], outs["fused"]), "aux vs fused must be bit-identical"


@pytest.mark.parametrize("name", sorted(SMALL_GEMM))
def test_small_layers_gemm_regime(orc, name):
    dev = device()
    shape, seed, counts = SMALL_GEMM[name]
    layer = synth.make_layer(shape, seed)
    dl = synth.layer_to(layer, dev)
    plans = {m: _plan(shape, max(counts), m, ffn.FORCE_GEMM) for m in MODES}
    for T in counts:
        x = synth.make_tokens(shape, T, seed, stream=T)
        ref = orc.forward(oracle_layer(layer), oracle_tokens(x))
        outs = {}
        for m, mf in plans.items():
            print(f"[gemm] {name} T={T} mode={m}", flush=True)
            got = run_gpu(mf, dl, x.to(dev))
            compare(orc, layer, x, got, tol_for(shape), ref=ref)
            outs[m] = got["out"]
        assert torch.equal(outs["aux"], outs["seq"]), "aux vs sequential must be bit-identical"
        assert torch.equal(outs["aux"], outs["fused"]), "aux vs fused must be bit-identical"


def test_force_gemm_rejected_for_other_storage():
    for shape in (synth.TINY, synth.DECODE_Q4, synth.LayerShape(160, 12, 3, 96, 64, "bf16", "bf16")):
        with pytest.raises(ffn.MoeFfnError) as ei:
            ffn.MoeFfn.for_shape(shape, max_tokens=4, flags=ffn.FORCE_GEMM)
        assert ei.value.status == ffn.ERR_UNSUPPORTED


# ---- the decode layer at full size ----------------------------------------------------

_LAYERS: dict = {}


def _decode_layer(shape, seed):
    """Drawn on the device with torch's seeded generator, copied to the host for the oracle."""
    key = (shape, seed)
    if key not in _LAYERS:
        dev = device()
        dl = synth.make_layer_device(shape, seed, dev)
        _LAYERS.clear()
        _LAYERS[key] = (dl, {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()})
    return _LAYERS[key]


FULL = {
    # name: (shape, seed, tokens, regime flags); the default regime switches to the
    # grouped GEMM above 16 tokens for bf16, so both regimes are also forced at
    # batches on the other side of it; routing runs in the gate/up launch up to 16
    # tokens (in its own launch where the batch's logits rows do not fit the gate/up
    # prologue) and in the batch launches above
    "decode_bf16_t1": (synth.DECODE_BF16, 1, 1, 0),
    "decode_bf16_t4": (synth.DECODE_BF16, 2, 4, 0),
    "decode_bf16_t5": (synth.DECODE_BF16, 2, 5, 0),
    "decode_bf16_t7": (synth.DECODE_BF16, 2, 7, 0),
    "decode_bf16_t8": (synth.DECODE_BF16, 2, 8, 0),
    "decode_bf16_t8_gemm": (synth.DECODE_BF16, 2, 8, ffn.FORCE_GEMM),
    "decode_bf16_t16": (synth.DECODE_BF16, 2, 16, 0),
    "decode_bf16_t17": (synth.DECODE_BF16, 2, 17, 0),
    "decode_bf16_t33": (synth.DECODE_BF16, 2, 33, 0),
    "decode_q4_t1": (synth.DECODE_Q4, 3, 1, 0),
    "decode_q4_t4": (synth.DECODE_Q4, 3, 4, 0),
    "decode_q4_t12": (synth.DECODE_Q4, 3, 12, 0),
    # one GPU's shard of the layer split eight ways inside every expert (I = I_s = 64)
    "decode_bf16_t1_tp8": (synth.DECODE_BF16_TP8, 7, 1, 0),
    "decode_bf16_t8_tp8": (synth.DECODE_BF16_TP8, 9, 8, 0),
}


@pytest.mark.parametrize("name", list(FULL))
def test_decode_layer_full_size(orc, name):
    dev = device()
    shape, seed, T, regime = FULL[name]
    dl, lc = _decode_layer(shape, seed)
    x = synth.make_tokens(shape, T, seed, stream=T)
    ref = orc.forward(oracle_layer(lc), oracle_tokens(x), nthreads=oracle_threads())
    outs = {}
    for m in MODES:
        print(f"[full] {name} mode={m}", flush=True)
        mf = _plan(shape, T, m, regime)
        got = run_gpu(mf, dl, x.to(dev))
        rep = compare(orc, lc, x, got, tol_for(shape), ref=ref)
        print(f"  {rep}", flush=True)
        outs[m] = got["out"]
        mf.close()
    assert torch.equal(outs["aux"], outs["seq"])
    assert torch.equal(outs["aux"], outs["fused"])


def test_decode_bf16_t128(orc):
    """Batch 128: the grouped-GEMM regime in every mode (bit-identical to each
    other) and the mat-vec regime forced, each against the oracle."""
    dev = device()
    shape, seed, T = synth.DECODE_BF16, 4, 128
    dl, lc = _decode_layer(shape, seed)
    x = synth.make_tokens(shape, T, seed, stream=T)
    ref = orc.forward(oracle_layer(lc), oracle_tokens(x), nthreads=oracle_threads())
    outs = {}
    for m in MODES:
        print(f"[full] decode_bf16_t128 gemm mode={m}", flush=True)
        mf = _plan(shape, T, m)
        got = run_gpu(mf, dl, x.to(dev))
        rep = compare(orc, lc, x, got, tol_for(shape), ref=ref)
        print(f"  {rep}", flush=True)
        assert rep["unique_experts"] > 200
        outs[m] = got["out"]
        mf.close()
    assert torch.equal(outs["aux"], outs["seq"])
    assert torch.equal(outs["aux"], outs["fused"])
    print("[full] decode_bf16_t128 matvec forced", flush=True)
    mf = _plan(shape, T, "aux", ffn.FORCE_MATVEC)
    rep = compare(orc, lc, x, run_gpu(mf, dl, x.to(dev)), tol_for(shape), ref=ref)
    print(f"  {rep}", flush=True)
    mf.close()


def _shard(layer: dict, r0: int, r1: int) -> dict:
    """Rows r0:r1 of the intermediate dimension of every expert and of the shared expert."""
    s = layer["shape"]
    out = dict(layer)
    out["shape"] = s.with_(inter=r1 - r0, shared_inter=r1 - r0)
    for name in ("gate", "up", "sh_gate", "sh_up"):
        out[name] = layer[name][..., r0:r1, :].contiguous()
    for name in ("down", "sh_down"):
        out[name] = layer[name][..., r0:r1].contiguous()
    return out


@pytest.mark.parametrize("T", [1, 8])
def test_tp8_shards_sum_to_the_layer(orc, T):
    """The layer split eight ways inside every expert (each shard holds 64 of the 512
    intermediate rows of every expert and of the shared expert, the router whole):
    every shard routes the same way, and the eight partial outputs, summed as an
    all-reduce would, give the whole layer's output within tolerance."""
    dev = device()
    shape, seed = synth.DECODE_BF16, 2
    dl, lc = _decode_layer(shape, seed)
    x = synth.make_tokens(shape, T, seed, stream=100 + T)
    ref = orc.forward(oracle_layer(lc), oracle_tokens(x), nthreads=oracle_threads())
    mf = _plan(shape, T, "fused")
    full = run_gpu(mf, dl, x.to(dev))
    mf.close()
    total = torch.zeros_like(full["out"], dtype=torch.float64)
    step = shape.inter // 8
    for r in range(8):
        print(f"[tp8] T={T} shard {r}", flush=True)
        sh = _shard(dl, r * step, (r + 1) * step)
        mf = _plan(sh["shape"], T, "fused")
        got = run_gpu(mf, sh, x.to(dev))
        mf.close()
        assert torch.equal(got["ids"], full["ids"]), f"shard {r} routes differently"
        total += got["out"].double()
    scale = float(np.max(np.abs(ref["out"])))
    err_sum = float(np.max(np.abs(total.numpy() - ref["out"])))
    err_full = float(np.max(np.abs(full["out"].double().numpy() - ref["out"])))
    print(f"  max |sum of shards - oracle| {err_sum:.3e}, max |layer - oracle| {err_full:.3e}, "
          f"scale {scale:.3e}", flush=True)
    assert err_sum <= TOL_LOWP * scale


SPLIT_JOIN_CASES = {
    # name: (shape, seed, tokens): the one-launch down + join against separate launches
    "tiny_fp32": (synth.TINY, 0, 3),
    "bf16_ragged_chunks": (synth.LayerShape(160, 12, 3, 96, 64, "bf16", "bf16"), 5, 6),
    "q4_wide": (synth.LayerShape(1024, 16, 4, 256, 128, "bf16", "q4"), 11, 6),
    "bf16_wide_rows": (synth.LayerShape(512, 16, 4, 2048, 1024, "bf16", "bf16"), 24, 5),
    "decode_bf16_t1": (synth.DECODE_BF16, 1, 1),
}


@pytest.mark.parametrize("name", sorted(SPLIT_JOIN_CASES))
def test_down_join_fused_matches_split(name):
    """One launch for down + join gives the same bits as two, in every shared mode."""
    dev = device()
    shape, seed, T = SPLIT_JOIN_CASES[name]
    dl = synth.layer_to(synth.make_layer(shape, seed), dev)
    x = synth.make_tokens(shape, T, seed, stream=T).to(dev)
    for m in MODES:
        print(f"[split-join] {name} T={T} mode={m}", flush=True)
        fused = run_gpu(_plan(shape, T, m, ffn.FORCE_MATVEC), dl, x)["out"]
        split = run_gpu(_plan(shape, T, m, ffn.FORCE_MATVEC | ffn.DEBUG_SPLIT_JOIN), dl, x)["out"]
        assert torch.equal(fused, split), f"mode {m}"


def test_many_pairs_top16(orc):
    """256 tokens x top-16 over 64 experts: 4096 pairs, big buckets."""
    dev = device()
    shape = synth.LayerShape(128, 64, 16, 64, 64, "bf16", "bf16")
    layer = synth.make_layer(shape, 25)
    x = synth.make_tokens(shape, 256, 25)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=256, flags=ffn.SHARED_FUSED)
    got = run_gpu(mf, synth.layer_to(layer, dev), x.to(dev))
    compare(orc, layer, x, got, tol_for(shape))


# ---- exact ties in the routing ----------------------------------------------------------

@pytest.mark.parametrize("T", [1, 9])
def test_exact_ties_go_to_the_lower_index(orc, T):
    """Duplicated router rows give bit-equal logits; the picks among them
    follow the expert index (and the oracle's fp64 ranking, tie for tie)."""
    dev = device()
    shape = synth.LayerShape(128, 16, 4, 64, 64, "bf16", "bf16")
    layer = dict(synth.make_layer(shape, 26))
    r = layer["router"].clone()
    r[9] = r[2]
    r[12] = r[4]
    r[5] = r[4]
    r[[2, 4, 5, 9, 12]] *= 4.0  # large enough to be picked for most tokens
    layer["router"] = r.contiguous()
    x = synth.make_tokens(shape, T, 26)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=T)
    got = run_gpu(mf, synth.layer_to(layer, dev), x.to(dev))
    ref = orc.forward(oracle_layer(layer), oracle_tokens(x))
    assert np.array_equal(got["ids"].numpy(), ref["ids"]), (got["ids"], ref["ids"])
    ids = got["ids"].numpy()
    for t in range(T):
        pos = {int(e): j for j, e in enumerate(ids[t])}
        for lo, hi in ((2, 9), (4, 5), (5, 12)):
            if lo in pos and hi in pos:
                assert pos[lo] < pos[hi], f"token {t}: expert {lo} must precede {hi}"
            assert not (hi in pos and lo not in pos), f"token {t}: {hi} picked without {lo}"


def test_all_logits_equal():
    """A zero router: every logit is +0, so the picks are experts 0..k-1 in
    order with equal weights, and a zero gate vector gives s = 1/2."""
    dev = device()
    shape = synth.LayerShape(128, 16, 4, 64, 64, "bf16", "bf16")
    layer = dict(synth.make_layer(shape, 27))
    layer["router"] = torch.zeros_like(layer["router"])
    layer["gate_vec"] = torch.zeros_like(layer["gate_vec"])
    x = synth.make_tokens(shape, 3, 27)
    got = run_gpu(ffn.MoeFfn.for_shape(shape, max_tokens=3), synth.layer_to(layer, dev), x.to(dev))
    assert torch.equal(got["ids"], torch.arange(4, dtype=torch.int32).repeat(3, 1))
    assert torch.all((got["weights"] - 0.25).abs() <= 1e-7)
    assert torch.all(got["gate"] == 0.5)


# ---- determinism, races, streams, capture ---------------------------------------------

@pytest.mark.parametrize("T", [8, 32])
def test_run_to_run_and_poisoned_workspace(T):
    dev = device()
    shape, seed = synth.DECODE_BF16, 2
    dl, _ = _decode_layer(shape, seed)
    x = synth.make_tokens(shape, T, seed, stream=T).to(dev)
    for m in MODES:
        mf = _plan(shape, T, m)
        ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
        first = run_gpu(mf, dl, x, ws=ws, poison=0)["out"]
        for i, pat in enumerate((0xFF, 0x7F, 0xA5, 0x00) * 5):
            again = run_gpu(mf, dl, x, ws=ws, poison=pat)["out"]
            assert torch.equal(first, again), f"mode {m}: run {i} with workspace fill {pat:#x} differs"
        mf.close()


@pytest.mark.parametrize("T", [8, 32])
@pytest.mark.parametrize("hook", ["delay_aux", "delay_main"])
def test_stream_order_with_injected_delay(hook, T):
    """A spin at the head of one branch must not change a single bit."""
    dev = device()
    shape, seed = synth.DECODE_BF16, 2
    dl, _ = _decode_layer(shape, seed)
    x = synth.make_tokens(shape, T, seed, stream=T).to(dev)
    base = run_gpu(_plan(shape, T, "seq"), dl, x)["out"]
    flag = ffn.DEBUG_DELAY_AUX if hook == "delay_aux" else ffn.DEBUG_DELAY_MAIN
    mf = _plan(shape, T, "aux", flag)
    for _ in range(3):
        assert torch.equal(run_gpu(mf, dl, x)["out"], base)


@pytest.mark.parametrize("T", [8, 32])
@pytest.mark.parametrize("mode", list(MODES))
def test_graph_capture_and_replay(mode, T):
    dev = device()
    shape, seed = synth.DECODE_BF16, 2
    dl, _ = _decode_layer(shape, seed)
    mf = _plan(shape, T, mode)
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    x_static = synth.make_tokens(shape, T, seed, stream=100).to(dev)
    out_static = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    mf.forward(dl, x_static, out_static, ws)  # first call: lazy set-up, never captured
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mf.forward(dl, x_static, out_static, ws)
    for i in range(4):
        xi = synth.make_tokens(shape, T, seed, stream=200 + i).to(dev)
        eager_out = torch.empty_like(out_static)
        eager_ws = torch.empty_like(ws)
        mf.forward(dl, xi, eager_out, eager_ws)
        torch.cuda.synchronize()
        x_static.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, eager_out), f"replay {i} differs from eager"


# ---- edge cases ----------------------------------------------------------------------

def test_in_place_fp32(orc):
    dev = device()
    shape = synth.TINY
    layer = synth.make_layer(shape, 0)
    dl = synth.layer_to(layer, dev)
    x = synth.make_tokens(shape, 3, 0, stream=3)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=3)
    ref = run_gpu(mf, dl, x.to(dev))["out"]
    buf = x.to(dev).clone()
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    mf.forward(dl, buf, buf, ws)
    torch.cuda.synchronize()
    assert torch.equal(buf.cpu(), ref)


def test_zero_tokens_is_a_no_op():
    dev = device()
    shape = synth.TINY
    dl = synth.layer_to(synth.make_layer(shape, 0), dev)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=4)
    x = torch.zeros(0, shape.hidden, dtype=torch.float32, device=dev)
    out = torch.full((1, shape.hidden), 7.0, device=dev)
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    mf.forward(dl, x, out, ws, n_tokens=0)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_max_tokens_256(orc):
    dev = device()
    shape = synth.LayerShape(128, 16, 2, 256, 64, "bf16", "bf16")
    layer = synth.make_layer(shape, 12)
    x = synth.make_tokens(shape, 256, 12)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=256)
    got = run_gpu(mf, synth.layer_to(layer, dev), x.to(dev))
    compare(orc, layer, x, got, tol_for(shape))


def test_max_tokens_256_gemm(orc):
    dev = device()
    shape = synth.LayerShape(128, 16, 2, 256, 128, "bf16", "bf16")
    layer = synth.make_layer(shape, 16)
    x = synth.make_tokens(shape, 256, 16)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=256)
    got = run_gpu(mf, synth.layer_to(layer, dev), x.to(dev))
    compare(orc, layer, x, got, tol_for(shape))


@pytest.mark.parametrize("regime", [ffn.FORCE_MATVEC, ffn.FORCE_GEMM])
def test_power_of_two_homogeneity(regime):
    """Doubling the down weights doubles every output exactly (in both regimes
    the activation feeding the down product does not depend on them)."""
    dev = device()
    shape = synth.LayerShape(256, 16, 4, 128, 128, "bf16", "bf16")
    layer = synth.make_layer(shape, 13)
    x = synth.make_tokens(shape, 5, 13).to(dev)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=5, flags=regime)
    base = run_gpu(mf, synth.layer_to(layer, dev), x)["out"]
    doubled = dict(layer)
    doubled["down"] = (layer["down"].float() * 2).to(torch.bfloat16)
    doubled["sh_down"] = (layer["sh_down"].float() * 2).to(torch.bfloat16)
    got = run_gpu(mf, synth.layer_to(doubled, dev), x)["out"]
    assert torch.equal(got, base * 2)


def test_q4_matches_dequantised_fp32():
    """The in-register 4-bit path against the fp32 path on exactly dequantised weights."""
    dev = device()
    shape = synth.LayerShape(512, 12, 3, 128, 96, "bf16", "q4")
    layer = synth.make_layer(shape, 14)
    x = synth.make_tokens(shape, 4, 14)
    q = run_gpu(ffn.MoeFfn.for_shape(shape, max_tokens=4), synth.layer_to(layer, dev), x.to(dev))

    def deq(name):
        w, s = layer[name], layer[name + "_scale"]
        lo = (w & 15).to(torch.float32) - 8
        hi = (w >> 4).to(torch.float32) - 8
        qv = torch.stack((lo, hi), dim=-1).flatten(-2)
        return qv * s.to(torch.float32).repeat_interleave(32, dim=-1)

    fshape = shape.with_(x_dtype="f32", w_dtype="f32")
    fl = {"shape": fshape, "router": layer["router"], "gate_vec": layer["gate_vec"]}
    for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        fl[n] = deq(n).contiguous()
        fl[n + "_scale"] = None
    f = run_gpu(ffn.MoeFfn.for_shape(fshape, max_tokens=4), synth.layer_to(fl, dev),
                x.to(torch.float32).to(dev))
    assert torch.equal(q["ids"], f["ids"])
    scale = f["out"].abs().max()
    assert (q["out"] - f["out"]).abs().max() <= 1e-4 * scale


def test_expert_permutation_equivariance():
    dev = device()
    shape = synth.LayerShape(256, 16, 4, 128, 64, "bf16", "q4")
    layer = synth.make_layer(shape, 15)
    x = synth.make_tokens(shape, 6, 15).to(dev)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=6)
    a = run_gpu(mf, synth.layer_to(layer, dev), x)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(shape.n_experts))
    pl = dict(layer)
    pl["router"] = layer["router"][perm].contiguous()
    for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale"):
        pl[n] = layer[n][perm].contiguous()
    b = run_gpu(mf, synth.layer_to(pl, dev), x)
    assert torch.equal(perm[b["ids"].long()].to(torch.int32), a["ids"])
    assert (a["out"] - b["out"]).abs().max() <= 1e-5 * a["out"].abs().max()
