"""GPU: the routing step's integer tables, read from the workspace after a forward,
equal their definition exactly (tests/routing_tables.py): every (token, slot) pair
bucketed once under its expert, buckets contiguous with their pairs ascending, the
used experts the distinct ids, the job records those of the buckets -- numbered in
order of first appearance when one workgroup routes the batch, ascending from the
batch launches.

Every routing placement is covered: the gate/up workgroups route the batch themselves
(up to 16 tokens: one token, the one-wave sort up to 64 pairs, the workgroup bitmap
above), a routing launch of its own (logits rows too many for the gate/up prologue),
and the three batch launches (above 16 tokens, and the grouped-GEMM regime).  The
ids in the workspace equal the debug ids, which match the oracle (near-tie rule) on
the tokens checked; the tables do not depend on the shared-expert mode.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from moe_decode_ffn_amd import ffn, synth
from tests.gpu_common import compare, device, oracle_threads, run_gpu, tol_for
from tests.helpers import oracle_layer, oracle_tokens
from tests.routing_tables import check_tables

pytestmark = pytest.mark.gpu

MODES = {"aux": ffn.SHARED_AUX, "seq": ffn.SHARED_SEQ, "fused": ffn.SHARED_FUSED}


def _tables(mf, ws, T):
    tab = mf.routing_tables(ws, T)
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in tab.items()}


def _check_call(orc, mf, layer_cpu, dl, x, n_check, modes=("fused",), batch_launches=None):
    """Runs the forward in each mode, checks the tables of each and their agreement,
    and the outputs of up to n_check tokens against the oracle."""
    dev = device()
    T = x.shape[0]
    tabs = {}
    for m in modes:
        plan = mf[m]
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
        ws.fill_(0xA5)  # poison: every table entry read must be written by this call
        got = run_gpu(plan, dl, x.to(dev), ws=ws)
        tab = _tables(plan, ws, T)
        ids = got["ids"].numpy()
        assert np.array_equal(tab["ids"].reshape(T, -1), ids), "workspace ids vs debug ids"
        assert np.array_equal(tab["weights"].reshape(T, -1), got["weights"].numpy())
        tabs[m] = (tab, got, check_tables(tab, ids))
    first = tabs[modes[0]][0]
    for m in modes[1:]:
        t = tabs[m][0]
        for key in ("n_used", "records", "pairs", "pair_expert", "ids"):
            assert np.array_equal(np.asarray(first[key]), np.asarray(t[key])), f"{key}: {modes[0]} vs {m}"
    got = tabs[modes[0]][1]
    orders = tabs[modes[0]][2]
    if batch_launches is not None:
        # records: ascending from the batch launches, first appearance from one workgroup
        # (the two coincide when the first appearances happen to be ascending)
        from tests.routing_tables import expert_order
        ids = got["ids"].numpy()
        same = expert_order(ids, "ascending") == expert_order(ids, "first")
        want = "ascending" if batch_launches else "first"
        assert orders[0] == want or same, f"record order {orders[0]}, expected {want}"
    idx = np.arange(T) if n_check >= T else np.sort(np.random.default_rng(T).choice(T, n_check, replace=False))
    sel = torch.from_numpy(idx)
    sub = {k: v[sel] for k, v in got.items()}
    ref = orc.forward(oracle_layer(layer_cpu), oracle_tokens(x[sel]), nthreads=oracle_threads())
    compare(orc, layer_cpu, x[sel], sub, tol_for(layer_cpu["shape"]), ref=ref)
    return first


@pytest.fixture(scope="module")
def decode_layer():
    dev = device()
    dl = synth.make_layer_device(synth.DECODE_BF16, 31, dev)
    lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    return dl, lc


@pytest.mark.parametrize("T", [1, 2, 8, 16, 17, 128, 2048])
def test_decode_layer_tables(orc, decode_layer, T):
    """Full-size layer (2048 hidden, 256 experts, top-8): gate/up-workgroup routing up to
    16 tokens (one token; 16..64 pairs: one-wave sort; 128 pairs: workgroup bitmap), the
    batch launches at 17, 128 and 2048 tokens."""
    dl, lc = decode_layer
    shape = synth.DECODE_BF16
    x = synth.make_tokens(shape, T, 31, stream=T)
    plans = {m: ffn.MoeFfn.for_shape(shape, max_tokens=T, flags=f) for m, f in MODES.items()}
    print(f"[tables] decode bf16 T={T}", flush=True)
    tab = _check_call(orc, plans, lc, dl, x, n_check=16, modes=tuple(MODES), batch_launches=T > 16)
    print(f"  used experts {tab['n_used']}", flush=True)
    for p in plans.values():
        p.close()


SMALL = {
    # name: (shape, seed, token counts, flags)
    "q4_decode_shape": (synth.DECODE_Q4, 32, (1, 4), 0),
    # 512 experts: 2 tokens route in gate/up, 12 tokens in the routing launch of their own
    "e512": (synth.LayerShape(128, 512, 8, 64, 32, "bf16", "bf16"), 33, (2, 12), 0),
    # 96 pairs (workgroup bitmap in the gate/up workgroups), 5 tokens of 4 experts
    # (buckets of several pairs through the one-wave sort)
    "top16": (synth.LayerShape(128, 24, 16, 64, 32, "bf16", "bf16"), 34, (6,), 0),
    "few_experts": (synth.LayerShape(96, 4, 2, 64, 32, "bf16", "bf16"), 35, (5, 40), 0),
    # the grouped-GEMM regime forced at small batches: a routing launch of its own (one
    # token, then buckets of several tokens), then the batch launches
    "gemm_forced": (synth.LayerShape(256, 12, 3, 128, 256, "bf16", "bf16"), 36, (1, 9, 40), ffn.FORCE_GEMM),
    # 512 experts x top-32: 32 and 96 pairs in the gate/up workgroups (one token; the
    # workgroup bitmap), 640 pairs through the batch launches
    "e512_k32": (synth.LayerShape(128, 512, 32, 128, 128, "bf16", "bf16"), 37, (1, 3, 20), 0),
    "fp32": (synth.LayerShape(288, 20, 4, 64, 96, "f32", "f32"), 38, (1, 11, 30), 0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_tables(orc, name):
    dev = device()
    shape, seed, counts, flags = SMALL[name]
    if shape.hidden >= 1024:
        dl = synth.make_layer_device(shape, seed, dev)
        lc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in dl.items()}
    else:
        lc = synth.make_layer(shape, seed)
        dl = synth.layer_to(lc, dev)
    plans = {m: ffn.MoeFfn.for_shape(shape, max_tokens=max(counts), flags=f | flags) for m, f in MODES.items()}
    for T in counts:
        x = synth.make_tokens(shape, T, seed, stream=T)
        print(f"[tables] {name} T={T}", flush=True)
        _check_call(orc, plans, lc, dl, x, n_check=16, modes=tuple(MODES))
    for p in plans.values():
        p.close()
