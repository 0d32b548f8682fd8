"""GPU: moe_ffn_forward_noalloc (the workspace in the library's static per-device array)
gives the bits of moe_ffn_forward (caller workspace) on the same inputs, call after
call, the second call of each pair with fewer tokens, and matches the oracle.  A plan
whose workspace exceeds the array is refused before anything runs."""
from __future__ import annotations

import pytest
import torch

from moe_decode_ffn_amd import ffn, synth
from tests.gpu_common import compare, device, oracle_threads, tol_for
from tests.helpers import oracle_layer, oracle_tokens

pytestmark = pytest.mark.gpu


def _dbg(T, shape, dev):
    return {"ids": torch.full((T, shape.top_k), -1, dtype=torch.int32, device=dev),
            "weights": torch.empty(T, shape.top_k, dtype=torch.float32, device=dev),
            "logits": torch.empty(T, shape.n_experts, dtype=torch.float32, device=dev),
            "gate": torch.empty(T, dtype=torch.float32, device=dev)}


def _pair(orc, mf, dl, lc, shape, T, seed):
    """One forward through each entry point; bit-identical outputs and ids, oracle parity."""
    dev = device()
    x = synth.make_tokens(shape, T, seed, stream=T).to(dev)
    ws = torch.empty(mf.workspace_bytes, dtype=torch.uint8, device=dev)
    ref_out = torch.full((T, shape.hidden), float("nan"), dtype=torch.float32, device=dev)
    ref_dbg = _dbg(T, shape, dev)
    mf.forward(dl, x, ref_out, ws, dbg=ref_dbg)
    out = torch.full((T, shape.hidden), float("nan"), dtype=torch.float32, device=dev)
    dbg = _dbg(T, shape, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ffn.moe_ffn_forward_noalloc(mf.plan, ffn.MoeFfn.tensors(dl, x, out, dbg), T, stream)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "noalloc vs caller workspace: outputs differ"
    assert torch.equal(dbg["ids"], ref_dbg["ids"]) and torch.equal(dbg["weights"], ref_dbg["weights"])
    got = {"out": out.cpu(), "ids": dbg["ids"].cpu(), "weights": dbg["weights"].cpu(),
           "logits": dbg["logits"].cpu(), "gate": dbg["gate"].cpu()}
    xc = x.cpu()
    ref = orc.forward(oracle_layer(lc), oracle_tokens(xc), nthreads=oracle_threads())
    compare(orc, lc, xc, got, tol_for(shape), ref=ref)


@pytest.mark.parametrize("mode", ["auto", "aux"])
def test_noalloc_decode_layer(orc, mode):
    """Full-size layer, batch 8 then batch 3 (mat-vec regime), then 128 and 40 tokens
    (grouped GEMM): two calls in a row on the same static workspace, the second smaller."""
    dev = device()
    shape = synth.DECODE_BF16
    dl = synth.make_layer_device(shape, 61, dev)
    lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    flags = {"auto": ffn.SHARED_AUTO, "aux": ffn.SHARED_AUX}[mode]
    for tmax, counts in ((8, (8, 3)), (128, (128, 40))):
        mf = ffn.MoeFfn.for_shape(shape, max_tokens=tmax, flags=flags)
        assert mf.workspace_bytes <= ffn.NOALLOC_WORKSPACE_BYTES
        for T in counts:
            print(f"[noalloc] decode {mode} T={T}", flush=True)
            _pair(orc, mf, dl, lc, shape, T, 61)
        mf.close()


@pytest.mark.parametrize("name", ["tiny", "q4"])
def test_noalloc_other_storage(orc, name):
    dev = device()
    if name == "tiny":
        shape, counts = synth.TINY, (3, 1)
        lc = synth.make_layer(shape, 62)
        dl = synth.layer_to(lc, dev)
    else:
        shape, counts = synth.DECODE_Q4, (4, 1)
        dl = synth.make_layer_device(shape, 63, dev)
        lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=counts[0])
    for T in counts:
        print(f"[noalloc] {name} T={T}", flush=True)
        _pair(orc, mf, dl, lc, shape, T, 62)
    mf.close()


def test_noalloc_refuses_a_plan_beyond_the_static_workspace():
    dev = device()
    shape = synth.DECODE_BF16
    mf = ffn.MoeFfn.for_shape(shape, max_tokens=2048)
    assert mf.workspace_bytes > ffn.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros(1, shape.hidden, dtype=torch.bfloat16, device=dev)
    out = torch.zeros(1, shape.hidden, dtype=torch.float32, device=dev)
    dl = synth.make_layer_device(shape, 64, dev)
    with pytest.raises(ffn.MoeFfnError) as e:
        ffn.moe_ffn_forward_noalloc(mf.plan, ffn.MoeFfn.tensors(dl, x, out), 1,
                                    torch.cuda.current_stream(dev).cuda_stream)
    assert e.value.status == ffn.ERR_WORKSPACE_TOO_SMALL
    mf.close()
