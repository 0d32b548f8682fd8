"""Host-side checks of the C ABI (no GPU needed, no compute calls).

The library must load, export every function include/moe_ffn.h declares, agree
with the binding's struct mirrors, validate plans and forward arguments before
touching the device, and size one workspace as shared region + routing region
+ the maximum (not the sum) of the sequential steps' scratch.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from moe_decode_ffn_amd import ffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ffn.LIBRARY):
        from moe_decode_ffn_amd.build import build_library
        build_library()
    return ffn.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ffn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_ffn_plan", "moe_ffn_forward", "moe_ffn_destroy", "moe_ffn_abi_version",
              "moe_ffn_status_string", "moe_ffn_plan_get_info"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", ffn.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s(\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        getattr(lib, n)  # resolvable through ctypes too


def test_abi_version_and_struct_mirrors(lib):
    assert lib.moe_ffn_abi_version() == ffn.ABI_VERSION
    assert lib.moe_ffn_struct_size(0) == ctypes.sizeof(ffn.Desc)
    assert lib.moe_ffn_struct_size(1) == ctypes.sizeof(ffn.Tensors)
    assert lib.moe_ffn_struct_size(2) == ctypes.sizeof(ffn.PlanInfo)
    assert lib.moe_ffn_struct_size(3) == ctypes.sizeof(ffn.RoutingLayout)
    assert lib.moe_ffn_struct_size(99) == 0


def test_status_strings(lib):
    for st in range(9):
        assert ffn.status_name(st) != "unknown status"
    assert ffn.status_name(1234) == "unknown status"


def desc(**kw):
    base = dict(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512, max_tokens=8,
                device=0, x_dtype=ffn.BF16, weight_dtype=ffn.BF16, flags=0, matvec_max_tokens=0,
                norm_eps=0.0)
    base.update(kw)
    return ffn.Desc(**base)


BAD_PLANS = [
    (dict(hidden=0), ffn.ERR_INVALID_ARG),
    (dict(n_experts=-1), ffn.ERR_INVALID_ARG),
    (dict(top_k=0), ffn.ERR_INVALID_ARG),
    (dict(top_k=300), ffn.ERR_INVALID_ARG),
    (dict(max_tokens=0), ffn.ERR_INVALID_ARG),
    (dict(device=-1), ffn.ERR_INVALID_ARG),
    (dict(x_dtype=7), ffn.ERR_INVALID_ARG),
    (dict(flags=0x4000), ffn.ERR_INVALID_ARG),
    (dict(flags=ffn.FORCE_GEMM | ffn.FORCE_MATVEC), ffn.ERR_INVALID_ARG),
    (dict(hidden=2050), ffn.ERR_UNSUPPORTED),
    (dict(inter=500), ffn.ERR_UNSUPPORTED),
    (dict(hidden=16384), ffn.ERR_UNSUPPORTED),
    (dict(n_experts=1024, top_k=8), ffn.ERR_UNSUPPORTED),
    (dict(top_k=33, n_experts=64), ffn.ERR_UNSUPPORTED),
    (dict(max_tokens=16385), ffn.ERR_UNSUPPORTED),
    (dict(x_dtype=ffn.F32, weight_dtype=ffn.BF16), ffn.ERR_UNSUPPORTED),
    (dict(x_dtype=ffn.BF16, weight_dtype=ffn.F32), ffn.ERR_UNSUPPORTED),
    # the grouped GEMM takes bf16 storage with sizes that are multiples of 128
    (dict(flags=ffn.FORCE_GEMM, weight_dtype=ffn.Q4_B32), ffn.ERR_UNSUPPORTED),
    (dict(flags=ffn.FORCE_GEMM, x_dtype=ffn.F32, weight_dtype=ffn.F32), ffn.ERR_UNSUPPORTED),
    (dict(flags=ffn.FORCE_GEMM, hidden=2080), ffn.ERR_UNSUPPORTED),
    (dict(flags=ffn.FORCE_GEMM, inter=544), ffn.ERR_UNSUPPORTED),
    (dict(flags=ffn.FORCE_GEMM, shared_inter=96), ffn.ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_PLANS)
def test_plan_rejects(lib, kw, status):
    with pytest.raises(ffn.MoeFfnError) as e:
        ffn.moe_ffn_plan(desc(**kw))
    assert e.value.status == status


def test_plan_null_arguments(lib):
    plan = ctypes.c_void_p(123)
    assert lib.moe_ffn_plan(None, ctypes.byref(plan), None) == ffn.ERR_INVALID_ARG
    assert plan.value is None  # cleared on failure
    assert lib.moe_ffn_plan(ctypes.byref(desc()), None, None) == ffn.ERR_INVALID_ARG
    lib.moe_ffn_destroy(None)  # no-op


def _logit_stride(E):
    return (E + 1 + 3) // 4 * 4


def _align(v):
    return (v + 255) // 256 * 256


def _batch_routing_ints(T, k, E):
    """Above 16 tokens the batch is ranked and bucketed by launches of their own,
    through global memory: per-expert totals, one count row per ranking workgroup
    (4 tokens up to 4096 tokens, 16 above: room for the most rows any batch up to
    T needs) and each pair's rank inside its workgroup."""
    if T <= 16:
        return 0
    W = max(1024, (T + 15) // 16) if T > 4096 else (T + 3) // 4
    return E + W * E + T * k


@pytest.mark.parametrize("T", [1, 8, 64, 128])
def test_workspace_is_shared_plus_routing_plus_max_of_phases(lib, T):
    H, E, k, I, Is = 2048, 256, 8, 512, 512
    plan, ws = ffn.moe_ffn_plan(desc(max_tokens=T))
    info = ffn.moe_ffn_plan_get_info(plan)
    ffn.moe_ffn_destroy(plan)
    shared = _align(T * Is * 4) + _align(T * H * 4)
    # routing region: gate, ids, weights, one 64-byte job record per expert, used-expert
    # count, bucketed pairs and their experts, logits [T][E+1 padded to a multiple of 4],
    # batch routing's ints
    routing = (_align(T * 4) + 2 * _align(T * k * 4) + _align(E * 64) + _align(16)
               + 2 * _align(T * k * 4) + _align(T * _logit_stride(E) * 4))
    routing += _align(_batch_routing_ints(T, k, E) * 4) if T > 16 else 0
    h, y = _align(T * k * I * 4), _align(T * k * H * 4)
    phases = {"gate/up": h, "down": h + y, "join": y}  # live scratch of each sequential step
    assert info.shared_region_bytes == shared
    assert info.routing_region_bytes == routing
    assert info.phase_region_bytes == max(phases.values())
    assert info.phase_region_bytes < sum(phases.values())
    assert ws == info.workspace_bytes == shared + routing + max(phases.values())


@pytest.mark.parametrize("x_dtype,w_dtype,xb", [(ffn.BF16, ffn.BF16, 2), (ffn.F32, ffn.F32, 4)])
def test_workspace_with_input_norm(lib, x_dtype, w_dtype, xb):
    # the normalised tokens (x_dtype) join the routing region; nothing else changes
    T, H = 8, 2048
    p0, ws0 = ffn.moe_ffn_plan(desc(max_tokens=T, x_dtype=x_dtype, weight_dtype=w_dtype))
    p1, ws1 = ffn.moe_ffn_plan(desc(max_tokens=T, x_dtype=x_dtype, weight_dtype=w_dtype,
                                    flags=ffn.INPUT_NORM | ffn.RESIDUAL, norm_eps=1e-6))
    i0, i1 = ffn.moe_ffn_plan_get_info(p0), ffn.moe_ffn_plan_get_info(p1)
    ffn.moe_ffn_destroy(p0)
    ffn.moe_ffn_destroy(p1)
    assert i1.routing_region_bytes == i0.routing_region_bytes + _align(T * H * xb)
    assert i1.shared_region_bytes == i0.shared_region_bytes
    assert i1.phase_region_bytes == i0.phase_region_bytes
    assert ws1 == ws0 + _align(T * H * xb)
    p2, ws2 = ffn.moe_ffn_plan(desc(max_tokens=T, x_dtype=x_dtype, weight_dtype=w_dtype,
                                    flags=ffn.RESIDUAL))
    ffn.moe_ffn_destroy(p2)
    assert ws2 == ws0  # the residual add needs no scratch


@pytest.mark.parametrize("eps", [-1e-6, float("nan"), float("inf"), -float("inf")])
def test_plan_rejects_bad_norm_eps(lib, eps):
    with pytest.raises(ffn.MoeFfnError) as e:
        ffn.moe_ffn_plan(desc(flags=ffn.INPUT_NORM, norm_eps=eps))
    assert e.value.status == ffn.ERR_INVALID_ARG
    p, _ = ffn.moe_ffn_plan(desc(flags=ffn.INPUT_NORM, norm_eps=0.0))  # eps 0 is allowed
    ffn.moe_ffn_destroy(p)


@pytest.mark.parametrize("T", [257, 4096, 8192])
def test_workspace_with_batch_routing(lib, T):
    # above 16 tokens the routing region also holds the bucketing launches' ints
    H, E, k, I, Is = 2048, 256, 8, 512, 512
    plan, ws = ffn.moe_ffn_plan(desc(max_tokens=T))
    info = ffn.moe_ffn_plan_get_info(plan)
    ffn.moe_ffn_destroy(plan)
    routing = (_align(T * 4) + 2 * _align(T * k * 4) + _align(E * 64) + _align(16)
               + 2 * _align(T * k * 4) + _align(T * _logit_stride(E) * 4) + _align(_batch_routing_ints(T, k, E) * 4))
    assert info.routing_region_bytes == routing
    assert ws == info.workspace_bytes == (_align(T * Is * 4) + _align(T * H * 4) + routing
                                          + _align(T * k * I * 4) + _align(T * k * H * 4))


@pytest.mark.parametrize("T", [1, 16, 300])
def test_routing_layout_lies_in_the_routing_region(lib, T):
    # the routing tables a forward leaves in the workspace: 256-byte aligned, disjoint,
    # inside the routing region (after the shared branch's region, before the phases)
    E, k = 256, 8
    plan, ws = ffn.moe_ffn_plan(desc(max_tokens=T))
    info = ffn.moe_ffn_plan_get_info(plan)
    lay = ffn.moe_ffn_plan_get_routing_layout(plan)
    ffn.moe_ffn_destroy(plan)
    assert (lay.record_ints, lay.record_pairs) == (16, 12)
    tables = [(lay.ids, T * k * 4), (lay.weights, T * k * 4), (lay.gate, T * 4), (lay.n_used, 4),
              (lay.records, E * lay.record_ints * 4), (lay.pairs, T * k * 4), (lay.pair_expert, T * k * 4)]
    lo, hi = info.shared_region_bytes, info.shared_region_bytes + info.routing_region_bytes
    for off, n in tables:
        assert off % 256 == 0 and lo <= off and off + n <= hi
    spans = sorted(tables)
    for (a, na), (b, _) in zip(spans, spans[1:]):
        assert a + na <= b
    with pytest.raises(ffn.MoeFfnError) as e:
        ffn.moe_ffn_plan_get_routing_layout(None)
    assert e.value.status == ffn.ERR_INVALID_ARG


def test_noalloc_refuses_before_any_device_call(lib):
    # a NULL plan, and a plan whose workspace exceeds the static array, are refused
    # before the entry point touches the device (this runs without a GPU)
    t = ffn.Tensors()
    assert lib.moe_ffn_forward_noalloc(None, ctypes.byref(t), 1, None) == ffn.ERR_INVALID_ARG
    plan, ws = ffn.moe_ffn_plan(desc(max_tokens=2048))
    assert ws > ffn.NOALLOC_WORKSPACE_BYTES
    assert lib.moe_ffn_forward_noalloc(plan, ctypes.byref(t), 1, None) == ffn.ERR_WORKSPACE_TOO_SMALL
    assert b"static workspace" in lib.moe_ffn_last_error()
    ffn.moe_ffn_destroy(plan)
    plan, ws = ffn.moe_ffn_plan(desc(max_tokens=128))  # the decode layer fits up to 128 tokens
    ffn.moe_ffn_destroy(plan)
    assert ws <= ffn.NOALLOC_WORKSPACE_BYTES


def test_plan_with_the_largest_expert_count_and_top_k(lib):
    # 512 experts x top-32 at 256 tokens: batch routing's ints for 8192 pairs
    E, k, T = 512, 32, 256
    plan, ws = ffn.moe_ffn_plan(desc(hidden=128, n_experts=E, top_k=k, inter=128, shared_inter=128,
                                     max_tokens=T))
    info = ffn.moe_ffn_plan_get_info(plan)
    ffn.moe_ffn_destroy(plan)
    routing = (_align(T * 4) + 2 * _align(T * k * 4) + _align(E * 64) + _align(16)
               + 2 * _align(T * k * 4) + _align(T * _logit_stride(E) * 4) + _align(_batch_routing_ints(T, k, E) * 4))
    assert info.routing_region_bytes == routing


def test_auto_mode_defaults(lib):
    plan, _ = ffn.moe_ffn_plan(desc())
    info = ffn.moe_ffn_plan_get_info(plan)
    ffn.moe_ffn_destroy(plan)
    # measured on MI355X: mat-vec kernels win up to 16 tokens, the grouped GEMM above;
    # folding the shared expert into the routed launches wins in both regimes
    assert info.matvec_max_tokens == 16
    assert info.shared_mode_matvec == ffn.SHARED_FUSED
    assert info.shared_mode_gemm == ffn.SHARED_FUSED
    for m in (ffn.SHARED_AUX, ffn.SHARED_SEQ, ffn.SHARED_FUSED):
        plan, _ = ffn.moe_ffn_plan(desc(flags=m))
        assert ffn.moe_ffn_plan_get_info(plan).shared_mode_matvec == m
        ffn.moe_ffn_destroy(plan)


# ---- forward argument validation: rejected before any HIP call ----------------------

class FakeTensors:
    """Distinct, 256-aligned, non-overlapping fake device addresses (never dereferenced)."""

    def __init__(self, q4=False):
        self.next = 1 << 40
        names = ["x", "w_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down",
                 "gate_vec", "out"]
        if q4:
            names += ["w_gate_scale", "w_up_scale", "w_down_scale", "sh_gate_scale",
                      "sh_up_scale", "sh_down_scale"]
        self.t = ffn.Tensors()
        for n in names:
            setattr(self.t, n, self.alloc())
        self.ws = self.alloc()

    def alloc(self):
        a = self.next
        self.next += 1 << 34  # far apart: no accidental overlap
        return a


@pytest.fixture
def plan(lib):
    p, ws = ffn.moe_ffn_plan(desc())
    yield p, ws
    ffn.moe_ffn_destroy(p)


def _fwd(lib, p, t, n, ws, wsb):
    return lib.moe_ffn_forward(p, ctypes.byref(t), n, ws, wsb, None)


def test_forward_validation(lib, plan):
    p, wsb = plan
    f = FakeTensors()
    assert lib.moe_ffn_forward(None, ctypes.byref(f.t), 1, f.ws, wsb, None) == ffn.ERR_INVALID_ARG
    assert _fwd(lib, p, f.t, -1, f.ws, wsb) == ffn.ERR_TOO_MANY_TOKENS
    assert _fwd(lib, p, f.t, 9, f.ws, wsb) == ffn.ERR_TOO_MANY_TOKENS
    assert _fwd(lib, p, f.t, 0, f.ws, wsb) == ffn.OK  # nothing to do
    assert _fwd(lib, p, f.t, 1, None, wsb) == ffn.ERR_INVALID_ARG
    assert _fwd(lib, p, f.t, 1, f.ws, wsb - 1) == ffn.ERR_WORKSPACE_TOO_SMALL
    assert _fwd(lib, p, f.t, 1, f.ws + 16, wsb) == ffn.ERR_MISALIGNED
    g = FakeTensors()
    g.t.w_up = g.t.w_up + 8
    assert _fwd(lib, p, g.t, 1, g.ws, wsb) == ffn.ERR_MISALIGNED
    g = FakeTensors()
    g.t.sh_down = None
    assert _fwd(lib, p, g.t, 1, g.ws, wsb) == ffn.ERR_INVALID_ARG
    g = FakeTensors(q4=True)  # scales on a bf16 plan
    assert _fwd(lib, p, g.t, 1, g.ws, wsb) == ffn.ERR_INVALID_ARG


def test_forward_validation_input_norm(lib, plan):
    p, wsb = plan
    f = FakeTensors()
    f.t.norm_weight = f.alloc()  # a norm weight on a plan without INPUT_NORM
    assert _fwd(lib, p, f.t, 1, f.ws, wsb) == ffn.ERR_INVALID_ARG
    pn, wsn = ffn.moe_ffn_plan(desc(flags=ffn.INPUT_NORM | ffn.RESIDUAL, norm_eps=1e-6))
    try:
        g = FakeTensors()  # INPUT_NORM without a norm weight
        assert _fwd(lib, pn, g.t, 1, g.ws, wsn) == ffn.ERR_INVALID_ARG
        g.t.norm_weight = g.alloc() + 4
        assert _fwd(lib, pn, g.t, 1, g.ws, wsn) == ffn.ERR_MISALIGNED
        g = FakeTensors()
        g.t.norm_weight = g.alloc()
        g.t.out = g.t.norm_weight  # out over the norm weight
        assert _fwd(lib, pn, g.t, 2, g.ws, wsn) == ffn.ERR_ALIAS
        g = FakeTensors()
        g.t.norm_weight = g.alloc()
        assert _fwd(lib, pn, g.t, 1, g.ws, wsn - 1) == ffn.ERR_WORKSPACE_TOO_SMALL
    finally:
        ffn.moe_ffn_destroy(pn)


def test_forward_aliasing(lib, plan):
    p, wsb = plan
    f = FakeTensors()
    f.t.out = f.t.x  # bf16 x: out (fp32) cannot alias x
    assert _fwd(lib, p, f.t, 2, f.ws, wsb) == ffn.ERR_ALIAS
    f = FakeTensors()
    f.t.out = f.t.w_down + 4096  # inside a weight tensor
    assert _fwd(lib, p, f.t, 2, f.ws, wsb) == ffn.ERR_ALIAS
    f = FakeTensors()
    f.t.out = f.ws + 256  # inside the workspace
    assert _fwd(lib, p, f.t, 2, f.ws, wsb) == ffn.ERR_ALIAS
    f = FakeTensors()
    f.t.x = f.ws + 512
    assert _fwd(lib, p, f.t, 2, f.ws, wsb) == ffn.ERR_ALIAS


def test_last_error_explains(lib, plan):
    p, wsb = plan
    f = FakeTensors()
    assert _fwd(lib, p, f.t, 1, f.ws, wsb - 1) == ffn.ERR_WORKSPACE_TOO_SMALL
    assert str(wsb) in lib.moe_ffn_last_error().decode()
