"""GPU parity of the optional input RMSNorm and residual add around the layer.

With INPUT_NORM the router launch normalises each token (one reciprocal RMS
per token, times the per-channel weight), uses it for the logits and writes it
once for both expert branches; with RESIDUAL the join adds the un-normalised
input to the layer's output.  Every case runs every shared-expert mode, which
must agree bit for bit, against the oracle with the same block.
"""
from __future__ import annotations

import pytest
import torch

from moe_decode_ffn_amd import ffn, synth
from tests.gpu_common import compare, device, oracle_threads, run_gpu, tol_for
from tests.helpers import oracle_layer, oracle_tokens

pytestmark = pytest.mark.gpu

MODES = {"aux": ffn.SHARED_AUX, "seq": ffn.SHARED_SEQ, "fused": ffn.SHARED_FUSED}
BLOCKS = {"norm+residual": (True, True), "norm": (True, False), "residual": (False, True)}

SMALL = {
    # name: (shape, seed, token counts, regime flags)
    "tiny_fp32": (synth.TINY, 0, (1, 3), 0),
    "bf16_ragged_chunks": (synth.LayerShape(160, 12, 3, 96, 64, "bf16", "bf16"), 5, (1, 5, 17), 0),
    "q4_ragged": (synth.LayerShape(192, 10, 3, 96, 160, "bf16", "q4"), 6, (1, 4, 9), 0),
    "fp32_two_slots": (synth.LayerShape(288, 20, 4, 64, 96, "f32", "f32"), 7, (2, 11), 0),
    "gemm_basic": (synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16"), 20, (1, 5, 17), ffn.FORCE_GEMM),
}


def _modes_agree(orc, layer, dl, shape, counts, regime, seed, tag):
    plans = {m: ffn.MoeFfn.for_layer(layer, max(counts), flags=f | regime) for m, f in MODES.items()}
    for T in counts:
        x = synth.make_tokens(shape, T, seed, stream=T)
        ref = orc.forward(oracle_layer(layer), oracle_tokens(x), nthreads=oracle_threads())
        outs = {}
        for m, mf in plans.items():
            print(f"[input-block] {tag} T={T} mode={m}", flush=True)
            got = run_gpu(mf, dl, x.to(dl["gate_vec"].device))
            rep = compare(orc, layer, x, got, tol_for(shape), ref=ref)
            outs[m] = got["out"]
        print(f"  {rep}", flush=True)
        assert torch.equal(outs["aux"], outs["seq"]), "aux vs sequential must be bit-identical"
        assert torch.equal(outs["aux"], outs["fused"]), "aux vs fused must be bit-identical"
    for mf in plans.values():
        mf.close()


@pytest.mark.parametrize("block", list(BLOCKS))
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layers(orc, name, block):
    dev = device()
    shape, seed, counts, regime = SMALL[name]
    norm, resid = BLOCKS[block]
    layer = synth.with_input_block(synth.make_layer(shape, seed), seed + 300, norm=norm, residual=resid)
    _modes_agree(orc, layer, synth.layer_to(layer, dev), shape, counts, regime, seed, f"{name} {block}")


FULL = {
    # name: (shape, seed, tokens): routing in the gate/up launch (1), the routing
    # launch (8), the grouped GEMM with the batch routing launches (33), 4-bit (4)
    "decode_bf16_t1": (synth.DECODE_BF16, 1, 1),
    "decode_bf16_t8": (synth.DECODE_BF16, 2, 8),
    "decode_bf16_t33": (synth.DECODE_BF16, 2, 33),
    "decode_q4_t4": (synth.DECODE_Q4, 3, 4),
}


@pytest.mark.parametrize("name", list(FULL))
def test_decode_layer_full_size(orc, name):
    dev = device()
    shape, seed, T = FULL[name]
    dl = synth.make_layer_device(shape, seed, dev)
    dl = synth.with_input_block(dl, seed + 400, eps=1e-6)
    lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    _modes_agree(orc, lc, dl, shape, (T,), 0, seed, name)


def test_eps_matters_for_small_tokens(orc):
    """Tokens of mean square ~1e-6 against eps = 1e-4: eps dominates the root."""
    dev = device()
    shape = synth.TINY
    layer = synth.with_input_block(synth.make_layer(shape, 31), 331, eps=1e-4)
    dl = synth.layer_to(layer, dev)
    x = synth.make_tokens(shape, 3, 31) * 1e-3
    for m, f in MODES.items():
        mf = ffn.MoeFfn.for_layer(layer, 3, flags=f)
        compare(orc, layer, x, run_gpu(mf, dl, x.to(dev)), tol_for(shape))
        mf.close()


@pytest.mark.parametrize("regime", [ffn.FORCE_MATVEC, ffn.FORCE_GEMM])
def test_residual_is_the_last_add(regime):
    """out(with residual) == fp32(x + out(without)) bit for bit, with the norm on."""
    dev = device()
    shape = synth.LayerShape(256, 16, 4, 128, 128, "bf16", "bf16")
    base = synth.make_layer(shape, 32)
    x = synth.make_tokens(shape, 5, 32).to(dev)
    with_r = synth.layer_to(synth.with_input_block(base, 332, residual=True), dev)
    without = synth.layer_to(synth.with_input_block(base, 332, residual=False), dev)
    a = run_gpu(ffn.MoeFfn.for_layer(with_r, 5, flags=regime), with_r, x)["out"]
    b = run_gpu(ffn.MoeFfn.for_layer(without, 5, flags=regime), without, x)["out"]
    assert torch.equal(a, x.float().cpu() + b)


def test_in_place_fp32_with_norm_and_residual(orc):
    """out may be x itself (fp32): the residual is read before the same element is written."""
    dev = device()
    shape = synth.LayerShape(288, 20, 4, 64, 96, "f32", "f32")
    layer = synth.with_input_block(synth.make_layer(shape, 33), 333)
    dl = synth.layer_to(layer, dev)
    x = synth.make_tokens(shape, 6, 33)
    for m, f in MODES.items():
        mf = ffn.MoeFfn.for_layer(layer, 6, flags=f)
        ref = run_gpu(mf, dl, x.to(dev))["out"]
        buf = x.to(dev).clone()
        ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
        mf.forward(dl, buf, buf, ws)
        torch.cuda.synchronize()
        assert torch.equal(buf.cpu(), ref), f"mode {m}"
        mf.close()


@pytest.mark.parametrize("mode", ["aux", "fused"])
def test_graph_capture_and_replay(mode):
    dev = device()
    shape, seed, T = synth.DECODE_BF16, 2, 8
    dl = synth.with_input_block(synth.make_layer_device(shape, seed, dev), 402)
    mf = ffn.MoeFfn.for_layer(dl, T, flags=MODES[mode])
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    x_static = synth.make_tokens(shape, T, seed, stream=100).to(dev)
    out_static = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    mf.forward(dl, x_static, out_static, ws)  # first call: lazy set-up, never captured
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mf.forward(dl, x_static, out_static, ws)
    for i in range(3):
        xi = synth.make_tokens(shape, T, seed, stream=200 + i).to(dev)
        eager_out = torch.empty_like(out_static)
        mf.forward(dl, xi, eager_out, torch.empty_like(ws))
        torch.cuda.synchronize()
        x_static.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, eager_out), f"replay {i} differs from eager"
    mf.close()
