"""GPU parity of large batches (prefill): above 16 tokens the batch is ranked by
its own launch (one wave per token, per-workgroup expert counts), the counts are
scanned per expert, and a third launch places every pair in its expert's bucket
(offset + the prefix of its workgroup + its rank inside it), through global memory.

Small layers are checked against the oracle on every token; the decode layer
at full size on a sample of tokens (each token's output depends on that token
alone, so the oracle runs on the sample).  Repeated runs must agree bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_decode_ffn_amd import ffn, synth
from tests.gpu_common import compare, device, oracle_threads, run_gpu, tol_for
from tests.helpers import oracle_layer, oracle_tokens

pytestmark = pytest.mark.gpu

MODES = {"aux": ffn.SHARED_AUX, "seq": ffn.SHARED_SEQ, "fused": ffn.SHARED_FUSED}

SMALL = {
    # name: (shape, seed, token counts, regime flags)
    "bf16_gemm": (synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16"), 40, (257, 300, 777), 0),
    "bf16_matvec": (synth.LayerShape(160, 12, 3, 96, 64, "bf16", "bf16"), 41, (300, 520), 0),
    "q4": (synth.LayerShape(192, 10, 3, 96, 160, "bf16", "q4"), 42, (400,), 0),
    "fp32": (synth.LayerShape(288, 20, 4, 64, 96, "f32", "f32"), 43, (300,), 0),
    # 16384 pairs over 64 experts: buckets of ~256 tokens, 64-token GEMM passes
    "bf16_big_buckets": (synth.LayerShape(128, 64, 16, 128, 128, "bf16", "bf16"), 44, (1024,), 0),
    "bf16_gemm_matvec_forced": (synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16"), 45, (300,),
                                ffn.FORCE_MATVEC),
    # the largest expert count and top-k: 512 experts (two per scanning thread), 32 picks a
    # token (128 pairs per ranking workgroup), 20 to 300 tokens: the batch launches
    "bf16_e512_k32": (synth.LayerShape(128, 512, 32, 128, 128, "bf16", "bf16"), 49, (20, 100, 300), 0),
    # the prefill GEMM's 192- and 256-token passes with its pipelined K loop running (it
    # needs at least 5 stages of 64: K >= 320 in gate/up (K = hidden 512) and in down
    # (K = inter 384)): mean buckets of 100 (192-token passes), 200 and 300 (256-token
    # passes; at 300 most buckets take a second, partial pass), and 525 (two or three
    # 256-token passes a bucket)
    "bf16_prefill_passes": (synth.LayerShape(512, 8, 2, 384, 384, "bf16", "bf16"), 50, (400, 800, 1200, 2100), 0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers_all_modes(orc, name):
    dev = device()
    shape, seed, counts, regime = SMALL[name]
    layer = synth.make_layer(shape, seed)
    dl = synth.layer_to(layer, dev)
    plans = {m: ffn.MoeFfn.for_shape(shape, max_tokens=max(counts), flags=f | regime) for m, f in MODES.items()}
    for T in counts:
        x = synth.make_tokens(shape, T, seed, stream=T)
        ref = orc.forward(oracle_layer(layer), oracle_tokens(x), nthreads=oracle_threads())
        outs = {}
        for m, mf in plans.items():
            print(f"[prefill] {name} T={T} mode={m}", flush=True)
            got = run_gpu(mf, dl, x.to(dev))
            rep = compare(orc, layer, x, got, tol_for(shape), ref=ref)
            outs[m] = got["out"]
        print(f"  {rep}", flush=True)
        assert torch.equal(outs["aux"], outs["seq"]), "aux vs sequential must be bit-identical"
        assert torch.equal(outs["aux"], outs["fused"]), "aux vs fused must be bit-identical"
    for mf in plans.values():
        mf.close()


def test_input_block_large_batch(orc):
    dev = device()
    shape = synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16")
    layer = synth.with_input_block(synth.make_layer(shape, 46), 346)
    dl = synth.layer_to(layer, dev)
    x = synth.make_tokens(shape, 600, 46)
    ref = orc.forward(oracle_layer(layer), oracle_tokens(x), nthreads=oracle_threads())
    outs = {}
    for m, f in MODES.items():
        print(f"[prefill] input block T=600 mode={m}", flush=True)
        mf = ffn.MoeFfn.for_layer(layer, 600, flags=f)
        got = run_gpu(mf, dl, x.to(dev))
        compare(orc, layer, x, got, tol_for(shape), ref=ref)
        outs[m] = got["out"]
        mf.close()
    assert torch.equal(outs["aux"], outs["seq"]) and torch.equal(outs["aux"], outs["fused"])


def test_max_tokens_16384(orc):
    dev = device()
    shape = synth.LayerShape(128, 16, 2, 128, 128, "bf16", "bf16")
    layer = synth.make_layer(shape, 47)
    x = synth.make_tokens(shape, 16384, 47)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=16384)
    print("[prefill] 16384 tokens", flush=True)
    got = run_gpu(mf, synth.layer_to(layer, dev), x.to(dev))
    compare(orc, layer, x, got, tol_for(shape))
    mf.close()


def _subset(got: dict, idx: np.ndarray) -> dict:
    return {k: v[torch.from_numpy(idx)] for k, v in got.items()}


FULL = {
    # name: (shape, seed, tokens, sampled tokens checked against the oracle)
    "decode_bf16_t2048": (synth.DECODE_BF16, 5, 2048, 48),
    "decode_q4_t512": (synth.DECODE_Q4, 6, 512, 32),
    # the prefill workloads as the benchmark runs them: mean buckets of 128 tokens
    # (192-token passes) and 512 tokens (256-token passes), K = 2048 and 512
    "prefill_bf16_t4096": (synth.DECODE_BF16, 9, 4096, 32),
    "prefill_bf16_t16384": (synth.DECODE_BF16, 10, 16384, 32),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(orc, name):
    """All modes bit-identical on every token; a sample of tokens against the oracle."""
    dev = device()
    shape, seed, T, n_check = FULL[name]
    dl = synth.make_layer_device(shape, seed, dev)
    lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    x = synth.make_tokens(shape, T, seed, stream=T)
    idx = np.sort(np.random.default_rng(seed).choice(T, n_check, replace=False))
    ref = orc.forward(oracle_layer(lc), oracle_tokens(x[torch.from_numpy(idx)]), nthreads=oracle_threads())
    outs = {}
    for m, f in MODES.items():
        print(f"[prefill] {name} mode={m}", flush=True)
        mf = ffn.MoeFfn.for_shape(shape, max_tokens=T, flags=f)
        got = run_gpu(mf, dl, x.to(dev))
        rep = compare(orc, lc, x[torch.from_numpy(idx)], _subset(got, idx), tol_for(shape), ref=ref)
        print(f"  {rep}", flush=True)
        outs[m] = got["out"]
        assert torch.all(torch.isfinite(got["out"]))
        mf.close()
    assert torch.equal(outs["aux"], outs["seq"])
    assert torch.equal(outs["aux"], outs["fused"])


def test_repeated_runs_give_the_same_bits():
    """Repeated large-batch runs, with the workspace poisoned in between, give the
    same bits (every workspace byte read is written in the same call)."""
    dev = device()
    shape, seed, T = synth.DECODE_BF16, 5, 2048
    dl = synth.make_layer_device(shape, seed, dev)
    x = synth.make_tokens(shape, T, seed, stream=7).to(dev)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=T)
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    first = run_gpu(mf, dl, x, ws=ws, poison=0)["out"]
    for i, pat in enumerate((0xFF, 0xA5, 0x00, 0x7F)):
        print(f"[prefill] repeat {i}", flush=True)
        assert torch.equal(run_gpu(mf, dl, x, ws=ws, poison=pat)["out"], first), f"run {i}"
    mf.close()


@pytest.mark.parametrize("T", [17, 512, 4096, 8200])
def test_router_logits_have_fp32_accuracy(orc, T):
    """Above 16 tokens the router is an MFMA GEMM over an exact three-way bf16 split
    of the fp32 weights (one, two or four 16-token tiles per workgroup splitting K four
    ways, and from 8192 tokens 64 tokens per workgroup over every row and all of K; 8200
    tokens end in a partial workgroup):
    its logits must be as close to the fp64 oracle as an fp32 dot product (a plain
    bf16 rounding of the weights would be off by ~1e-3)."""
    dev = device()
    shape, seed = synth.DECODE_BF16, 8
    dl = synth.make_layer_device(shape, seed, dev)
    lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    x = synth.make_tokens(shape, T, seed)
    idx = np.arange(0, T, max(1, T // 32))
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=T)
    got = run_gpu(mf, dl, x.to(dev))
    ref = orc.forward(oracle_layer(lc), oracle_tokens(x[torch.from_numpy(idx)]), nthreads=oracle_threads())
    err = np.max(np.abs(got["logits"][torch.from_numpy(idx)].double().numpy() - ref["logits"]))
    gerr = np.max(np.abs(got["gate"][torch.from_numpy(idx)].double().numpy() - ref["gate"]))
    print(f"  max |logit error| {err:.3e}, max |gate error| {gerr:.3e}", flush=True)
    assert err <= 1e-5 and gerr <= 1e-6
    mf.close()


def test_prefill_gemm_gives_the_bits_of_the_small_gemm():
    """The prefill GEMM takes over from a mean bucket of 32 tokens (128 tokens of this
    layer: 12 experts, top-3); it walks K in the same order with the same lane mapping
    as the smaller grouped GEMM, so the 127 tokens shared by a 127- and a 128-token
    batch (one below, one at the switch) get the same bits."""
    dev = device()
    shape = synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16")
    dl = synth.layer_to(synth.make_layer(shape, 48), dev)
    x = synth.make_tokens(shape, 128, 48).to(dev)
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=128)
    small = run_gpu(mf, dl, x[:127].contiguous())
    big = run_gpu(mf, dl, x)
    assert torch.equal(small["ids"], big["ids"][:127])
    assert torch.equal(small["out"], big["out"][:127])
    mf.close()
