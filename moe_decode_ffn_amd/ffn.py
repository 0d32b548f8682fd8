"""Python binding of libmoe_ffn.so (include/moe_ffn.h): argument marshalling only.

The entry points keep the C names (``moe_ffn_plan``, ``moe_ffn_forward``,
``moe_ffn_destroy`` ...).  Every step of the layer runs in the HIP library;
PyTorch is used here only for device pointers (``data_ptr``) and the stream
handle.  If the library is missing, loading raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "lib", "libmoe_ffn.so")

ABI_VERSION = 2
NOALLOC_WORKSPACE_BYTES = 16 << 20  # MOE_FFN_NOALLOC_WORKSPACE_BYTES

# moe_ffn_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL = 0, 1, 2, 3
ERR_MISALIGNED, ERR_ALIAS, ERR_TOO_MANY_TOKENS, ERR_HIP, ERR_WRONG_DEVICE = 4, 5, 6, 7, 8
# moe_ffn_dtype
F32, BF16, Q4_B32 = 0, 1, 2
# flags
SHARED_AUTO, SHARED_AUX, SHARED_SEQ, SHARED_FUSED, SHARED_MASK = 0x0, 0x1, 0x2, 0x3, 0x3
FORCE_MATVEC, FORCE_GEMM = 0x10, 0x20
INPUT_NORM, RESIDUAL = 0x1000, 0x2000
DEBUG_DELAY_AUX, DEBUG_DELAY_MAIN, DEBUG_SPLIT_JOIN = 0x100, 0x200, 0x400
# moe_ffn_kernel_id
KERNELS = ("router", "route", "gate_up", "down", "sh_gate_up", "sh_down", "join", "gg_gate_up",
           "gg_down", "down_join", "bucket")
K_COUNT = len(KERNELS)

DTYPES = {"f32": F32, "bf16": BF16, "q4": Q4_B32}


class MoeFfnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_name(status)} ({status}): {detail}")


class Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("device", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("matvec_max_tokens", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


_P = ctypes.c_void_p


class Tensors(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "x", "w_router", "w_gate", "w_up", "w_down", "w_gate_scale", "w_up_scale",
        "w_down_scale", "sh_gate", "sh_up", "sh_down", "sh_gate_scale", "sh_up_scale",
        "sh_down_scale", "gate_vec", "out", "dbg_topk_ids", "dbg_topk_weights", "dbg_logits",
        "dbg_shared_gate", "norm_weight")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_size_t), ("shared_region_bytes", ctypes.c_size_t),
                ("routing_region_bytes", ctypes.c_size_t), ("phase_region_bytes", ctypes.c_size_t),
                ("matvec_max_tokens", ctypes.c_int32), ("shared_mode_matvec", ctypes.c_uint32),
                ("shared_mode_gemm", ctypes.c_uint32)]


class RoutingLayout(ctypes.Structure):
    _fields_ = [("ids", ctypes.c_size_t), ("weights", ctypes.c_size_t), ("gate", ctypes.c_size_t),
                ("n_used", ctypes.c_size_t), ("records", ctypes.c_size_t), ("pairs", ctypes.c_size_t),
                ("pair_expert", ctypes.c_size_t), ("record_ints", ctypes.c_int32),
                ("record_pairs", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Loads the HIP library (once); raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m moe_decode_ffn_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.moe_ffn_abi_version.restype = ctypes.c_int32
    lib.moe_ffn_status_string.restype = ctypes.c_char_p
    lib.moe_ffn_status_string.argtypes = [ctypes.c_int32]
    lib.moe_ffn_last_error.restype = ctypes.c_char_p
    lib.moe_ffn_struct_size.restype = ctypes.c_size_t
    lib.moe_ffn_struct_size.argtypes = [ctypes.c_int32]
    lib.moe_ffn_plan.restype = ctypes.c_int32
    lib.moe_ffn_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_ffn_plan_get_info.restype = ctypes.c_int32
    lib.moe_ffn_plan_get_info.argtypes = [_P, ctypes.POINTER(PlanInfo)]
    lib.moe_ffn_plan_get_routing_layout.restype = ctypes.c_int32
    lib.moe_ffn_plan_get_routing_layout.argtypes = [_P, ctypes.POINTER(RoutingLayout)]
    lib.moe_ffn_forward.restype = ctypes.c_int32
    lib.moe_ffn_forward.argtypes = [_P, ctypes.POINTER(Tensors), ctypes.c_int32, _P,
                                    ctypes.c_size_t, _P]
    lib.moe_ffn_forward_noalloc.restype = ctypes.c_int32
    lib.moe_ffn_forward_noalloc.argtypes = [_P, ctypes.POINTER(Tensors), ctypes.c_int32, _P]
    lib.moe_ffn_destroy.restype = None
    lib.moe_ffn_destroy.argtypes = [_P]
    lib.moe_ffn_profile_enable.restype = ctypes.c_int32
    lib.moe_ffn_profile_enable.argtypes = [_P, ctypes.c_int32]
    lib.moe_ffn_profile_read.restype = ctypes.c_int32
    lib.moe_ffn_profile_read.argtypes = [_P, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int64)]
    if lib.moe_ffn_abi_version() != ABI_VERSION:
        raise ImportError("libmoe_ffn.so ABI version mismatch")
    for which, st in enumerate((Desc, Tensors, PlanInfo, RoutingLayout)):
        if lib.moe_ffn_struct_size(which) != ctypes.sizeof(st):
            raise ImportError(f"struct mirror {st.__name__} does not match the library")
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().moe_ffn_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MoeFfnError(status, where, load().moe_ffn_last_error().decode())


# ---- the C entry points --------------------------------------------------------

def moe_ffn_abi_version() -> int:
    return load().moe_ffn_abi_version()


def moe_ffn_plan(desc: Desc) -> tuple[int, int]:
    """Returns (plan handle, workspace bytes)."""
    plan = _P()
    ws = ctypes.c_size_t(0)
    _check(load().moe_ffn_plan(ctypes.byref(desc), ctypes.byref(plan), ctypes.byref(ws)), "moe_ffn_plan")
    return plan.value, ws.value


def moe_ffn_plan_get_info(plan: int) -> PlanInfo:
    info = PlanInfo()
    _check(load().moe_ffn_plan_get_info(plan, ctypes.byref(info)), "moe_ffn_plan_get_info")
    return info


def moe_ffn_plan_get_routing_layout(plan: int) -> RoutingLayout:
    lay = RoutingLayout()
    _check(load().moe_ffn_plan_get_routing_layout(plan, ctypes.byref(lay)),
           "moe_ffn_plan_get_routing_layout")
    return lay


def moe_ffn_forward(plan: int, tensors: Tensors, n_tokens: int, workspace: int,
                    workspace_bytes: int, stream: int) -> None:
    _check(load().moe_ffn_forward(plan, ctypes.byref(tensors), n_tokens, workspace,
                                  workspace_bytes, stream), "moe_ffn_forward")


def moe_ffn_forward_noalloc(plan: int, tensors: Tensors, n_tokens: int, stream: int) -> None:
    _check(load().moe_ffn_forward_noalloc(plan, ctypes.byref(tensors), n_tokens, stream),
           "moe_ffn_forward_noalloc")


def moe_ffn_destroy(plan: int) -> None:
    load().moe_ffn_destroy(plan)


def moe_ffn_profile_enable(plan: int, enable: bool) -> None:
    _check(load().moe_ffn_profile_enable(plan, 1 if enable else 0), "moe_ffn_profile_enable")


def moe_ffn_profile_read(plan: int) -> dict:
    ms = (ctypes.c_double * K_COUNT)()
    n = (ctypes.c_int64 * K_COUNT)()
    _check(load().moe_ffn_profile_read(plan, ms, n), "moe_ffn_profile_read")
    return {KERNELS[i]: (ms[i], n[i]) for i in range(K_COUNT)}


# ---- convenience wrapper over torch device tensors (still marshalling only) ----------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class MoeFfn:
    """A plan plus the bookkeeping to call it with torch tensors.

    ``layer`` dicts use the keys router, gate, up, down, sh_gate, sh_up, sh_down,
    gate_vec and, for 4-bit storage, <name>_scale; with the INPUT_NORM flag also
    norm_w (fp32 [H]).
    """

    def __init__(self, hidden, n_experts, top_k, inter, shared_inter, max_tokens, x_dtype="bf16",
                 w_dtype="bf16", flags=SHARED_AUTO, device=0, matvec_max_tokens=0, norm_eps=0.0):
        self.desc = Desc(hidden, n_experts, top_k, inter, shared_inter, max_tokens, device,
                         DTYPES[x_dtype], DTYPES[w_dtype], flags, matvec_max_tokens, norm_eps)
        self.plan, self.workspace_bytes = moe_ffn_plan(self.desc)

    @classmethod
    def for_shape(cls, shape, max_tokens, **kw):
        return cls(shape.hidden, shape.n_experts, shape.top_k, shape.inter, shape.shared_inter,
                   max_tokens, shape.x_dtype, shape.w_dtype, **kw)

    @classmethod
    def for_layer(cls, layer: dict, max_tokens, flags=SHARED_AUTO, **kw):
        """A plan for a layer dict; its norm_w / norm_eps / residual keys add the
        INPUT_NORM / RESIDUAL flags and the eps."""
        if layer.get("norm_w") is not None:
            flags |= INPUT_NORM
            kw.setdefault("norm_eps", float(layer.get("norm_eps", 0.0)))
        if layer.get("residual"):
            flags |= RESIDUAL
        return cls.for_shape(layer["shape"], max_tokens, flags=flags, **kw)

    def info(self) -> PlanInfo:
        return moe_ffn_plan_get_info(self.plan)

    def routing_layout(self) -> RoutingLayout:
        return moe_ffn_plan_get_routing_layout(self.plan)

    def routing_tables(self, workspace, n_tokens: int) -> dict:
        """Views of the routing tables a forward of n_tokens left in `workspace` (a uint8
        tensor): ids, weights, gate, n_used, records [U, record_ints], pairs, pair_expert."""
        import torch
        lay = self.routing_layout()
        npair = n_tokens * self.desc.top_k

        def view(off, n, dtype):
            return workspace[off:off + 4 * n].view(dtype)

        n_used = int(view(lay.n_used, 1, torch.int32).item())
        n_rec = max(0, min(n_used, self.desc.n_experts))
        return {"ids": view(lay.ids, npair, torch.int32), "weights": view(lay.weights, npair, torch.float32),
                "gate": view(lay.gate, n_tokens, torch.float32), "n_used": n_used,
                "records": view(lay.records, n_rec * lay.record_ints, torch.int32).reshape(n_rec, lay.record_ints),
                "pairs": view(lay.pairs, npair, torch.int32),
                "pair_expert": view(lay.pair_expert, npair, torch.int32),
                "record_pairs": lay.record_pairs}

    def close(self) -> None:
        if self.plan:
            moe_ffn_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def tensors(layer: dict, x, out, dbg: Optional[dict] = None) -> Tensors:
        dbg = dbg or {}
        return Tensors(
            _ptr(x), _ptr(layer["router"]), _ptr(layer["gate"]), _ptr(layer["up"]),
            _ptr(layer["down"]), _ptr(layer.get("gate_scale")), _ptr(layer.get("up_scale")),
            _ptr(layer.get("down_scale")), _ptr(layer["sh_gate"]), _ptr(layer["sh_up"]),
            _ptr(layer["sh_down"]), _ptr(layer.get("sh_gate_scale")),
            _ptr(layer.get("sh_up_scale")), _ptr(layer.get("sh_down_scale")),
            _ptr(layer["gate_vec"]), _ptr(out), _ptr(dbg.get("ids")), _ptr(dbg.get("weights")),
            _ptr(dbg.get("logits")), _ptr(dbg.get("gate")), _ptr(layer.get("norm_w")))

    def forward(self, layer: dict, x, out, workspace, stream=None, dbg: Optional[dict] = None,
                n_tokens: Optional[int] = None) -> None:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        handle = stream if isinstance(stream, int) else stream.cuda_stream
        t = self.tensors(layer, x, out, dbg)
        moe_ffn_forward(self.plan, t, x.shape[0] if n_tokens is None else n_tokens,
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(), handle)

    def profile_enable(self, on: bool = True) -> None:
        moe_ffn_profile_enable(self.plan, on)

    def profile_read(self) -> dict:
        return moe_ffn_profile_read(self.plan)
