"""CPU oracle for the MoE decode FFN layer with a gated shared expert.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It never imports the GPU
package, and the GPU package never imports it.

Two independent implementations of the same definition live here:

* ``forward`` drives the plain C fp64 oracle (``moe_ffn_oracle.c``): one token
  at a time, only the k selected experts, in the order of the definition.
* ``brute_force`` is a numpy fp64 twin written separately: it evaluates *every*
  expert on every token, then selects and combines.  Agreement of the two on
  small layers checks selection, renormalisation and the final identity
  out = sum_j w_j E_{ids_j}(x) + sigmoid(wg . x) S(x), with the optional input
  RMSNorm (x = RMSNorm(x0) * wn) and residual (out += x0) around it.

The layer definition, its citations and the 4-bit storage reading are in the C
file's header comment.  Inputs are plain numpy arrays:

  x         float32 [T,H] or uint16 [T,H] (bf16 bits)
  router    float32 [E,H]           gate_vec float32 [H]
  gate, up  float32 | uint16 (bf16 bits) [E,I,H]  or uint8 [E,I,H/2] (4-bit)
  down      ...                      [E,H,I]       or uint8 [E,H,I/2]
  sh_gate, sh_up [I_s,H]; sh_down [H,I_s] (same storage as the experts)
  *_scale   uint16 fp16 bits [..., K/32] for 4-bit storage, else None
  norm_w    float32 [H] or None (input RMSNorm weight; norm_eps its epsilon)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "moe_ffn_oracle.c")
LIBRARY = os.path.join(HERE, "libmoe_ffn_oracle.so")

KIND_F32, KIND_BF16, KIND_Q4 = 0, 1, 2
_KIND = {"f32": KIND_F32, "bf16": KIND_BF16, "q4": KIND_Q4}


def compile_library(source: str = SOURCE, output: str = LIBRARY) -> str:
    """gcc -O2 -fopenmp -shared; strict IEEE (no -ffast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Werror", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return output


class _Matrix(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("data", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rows", ctypes.c_long), ("cols", ctypes.c_long)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int),
                ("inter", ctypes.c_int), ("shared_inter", ctypes.c_int), ("x_kind", ctypes.c_int),
                ("x", ctypes.c_void_p), ("router", ctypes.c_void_p),
                ("gate", _Matrix), ("up", _Matrix), ("down", _Matrix),
                ("sh_gate", _Matrix), ("sh_up", _Matrix), ("sh_down", _Matrix),
                ("gate_vec", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("norm_eps", ctypes.c_double), ("residual", ctypes.c_int)]


class Oracle:
    """A loaded oracle library (the built one, or any compiled variant)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            compile_library(SOURCE, path)
        self.path = path
        self.lib = ctypes.CDLL(path)
        self.lib.orc_forward.restype = ctypes.c_int
        self.lib.orc_forward.argtypes = [ctypes.POINTER(_Layer), ctypes.c_long, ctypes.c_int,
                                         ctypes.c_void_p] + [ctypes.c_void_p] * 7
        self.lib.orc_bf16_value.restype = ctypes.c_double
        self.lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        self.lib.orc_f16_value.restype = ctypes.c_double
        self.lib.orc_f16_value.argtypes = [ctypes.c_uint16]
        self.lib.orc_matrix_decode.restype = None
        self.lib.orc_matrix_decode.argtypes = [ctypes.POINTER(_Matrix), ctypes.c_long,
                                               ctypes.c_long, ctypes.c_void_p]

    # -- decoders (exposed for the pins) -----------------------------------
    def bf16_value(self, bits: int) -> float:
        return self.lib.orc_bf16_value(bits)

    def f16_value(self, bits: int) -> float:
        return self.lib.orc_f16_value(bits)

    def decode_matrix(self, w: np.ndarray, scale: np.ndarray | None, kind: str) -> np.ndarray:
        """Decode a 2-D stored matrix (rows x logical cols) to float64 via the C decoder."""
        w = np.ascontiguousarray(w)
        rows = w.shape[0]
        cols = w.shape[1] * (2 if kind == "q4" else 1)
        m = _matrix(w, scale, kind, rows, cols)
        dst = np.empty((rows, cols), dtype=np.float64)
        self.lib.orc_matrix_decode(ctypes.byref(m), 0, rows, dst.ctypes.data)
        return dst

    # -- the layer ----------------------------------------------------------
    def forward(self, layer: "OracleLayer", x: np.ndarray, nthreads: int = 1,
                forced_ids: np.ndarray | None = None) -> dict:
        x = np.ascontiguousarray(x)
        T = x.shape[0]
        H, E, K = layer.hidden, layer.n_experts, layer.top_k
        L = layer.ctypes_layer(x)
        res = {
            "out": np.zeros((T, H)), "routed": np.zeros((T, H)), "shared": np.zeros((T, H)),
            "ids": np.zeros((T, K), dtype=np.int32), "weights": np.zeros((T, K)),
            "logits": np.zeros((T, E)), "gate": np.zeros(T),
        }
        fids = None
        if forced_ids is not None:
            fids = np.ascontiguousarray(forced_ids, dtype=np.int32)
            assert fids.shape == (T, K)
        rc = self.lib.orc_forward(
            ctypes.byref(L), T, nthreads, None if fids is None else fids.ctypes.data,
            res["out"].ctypes.data, res["routed"].ctypes.data, res["shared"].ctypes.data,
            res["ids"].ctypes.data, res["weights"].ctypes.data, res["logits"].ctypes.data,
            res["gate"].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return res


def _matrix(w, scale, kind, rows, cols) -> _Matrix:
    m = _Matrix()
    m.kind = _KIND[kind]
    m.data = w.ctypes.data
    m.scale = None if scale is None else scale.ctypes.data
    m.rows, m.cols = rows, cols
    return m


@dataclass
class OracleLayer:
    """A layer's weights as plain numpy arrays (see the module docstring)."""
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    x_kind: str
    w_kind: str
    router: np.ndarray
    gate: np.ndarray
    up: np.ndarray
    down: np.ndarray
    sh_gate: np.ndarray
    sh_up: np.ndarray
    sh_down: np.ndarray
    gate_vec: np.ndarray
    gate_scale: np.ndarray | None = None
    up_scale: np.ndarray | None = None
    down_scale: np.ndarray | None = None
    sh_gate_scale: np.ndarray | None = None
    sh_up_scale: np.ndarray | None = None
    sh_down_scale: np.ndarray | None = None
    norm_w: np.ndarray | None = None      # float32 [H]: RMSNorm of the input first
    norm_eps: float = 0.0
    residual: bool = False                # out = x + layer output

    def __post_init__(self):
        for name in ("router", "gate", "up", "down", "sh_gate", "sh_up", "sh_down", "gate_vec",
                     "gate_scale", "up_scale", "down_scale", "sh_gate_scale", "sh_up_scale",
                     "sh_down_scale", "norm_w"):
            v = getattr(self, name)
            if v is not None:
                setattr(self, name, np.ascontiguousarray(v))
        assert self.router.dtype == np.float32 and self.gate_vec.dtype == np.float32
        assert self.norm_w is None or self.norm_w.dtype == np.float32

    def ctypes_layer(self, x: np.ndarray) -> _Layer:
        H, E, I, Is = self.hidden, self.n_experts, self.inter, self.shared_inter
        want = np.float32 if self.x_kind == "f32" else np.uint16
        if x.dtype != want or x.ndim != 2 or x.shape[1] != H:
            raise ValueError("token array does not match the layer")
        L = _Layer()
        L.hidden, L.n_experts, L.top_k, L.inter, L.shared_inter = H, E, self.top_k, I, Is
        L.x_kind = _KIND[self.x_kind]
        L.x = x.ctypes.data
        L.router = self.router.ctypes.data
        k = self.w_kind
        L.gate = _matrix(self.gate, self.gate_scale, k, E * I, H)
        L.up = _matrix(self.up, self.up_scale, k, E * I, H)
        L.down = _matrix(self.down, self.down_scale, k, E * H, I)
        L.sh_gate = _matrix(self.sh_gate, self.sh_gate_scale, k, Is, H)
        L.sh_up = _matrix(self.sh_up, self.sh_up_scale, k, Is, H)
        L.sh_down = _matrix(self.sh_down, self.sh_down_scale, k, H, Is)
        L.gate_vec = self.gate_vec.ctypes.data
        L.norm_w = None if self.norm_w is None else self.norm_w.ctypes.data
        L.norm_eps = float(self.norm_eps)
        L.residual = 1 if self.residual else 0
        self._keepalive = (x,)
        return L


# ---------------------------------------------------------------------------
# numpy brute-force twin
# ---------------------------------------------------------------------------

def np_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (the bits are the top half of a float32)."""
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_f16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64, from the binary16 fields."""
    bits = bits.astype(np.int64)
    sign = np.where(bits >> 15, -1.0, 1.0)
    expo = (bits >> 10) & 31
    frac = (bits & 1023).astype(np.float64)
    normal = np.ldexp(1024.0 + frac, (expo - 25).astype(np.int32))
    sub = np.ldexp(frac, -24)
    val = np.where(expo == 0, sub, normal)
    val = np.where(expo == 31, np.where(frac == 0, np.inf, np.nan), val)
    return sign * val


def np_q4(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """[..., K/2] nibble bytes + [..., K/32] fp16 scales -> float64 [..., K]."""
    lo = (packed & 15).astype(np.int64) - 8
    hi = (packed >> 4).astype(np.int64) - 8
    q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.float64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    scales = np.repeat(np_f16(scale_bits), 32, axis=-1)
    return scales * q


def np_decode(w: np.ndarray, scale: np.ndarray | None, kind: str) -> np.ndarray:
    if kind == "f32":
        return w.astype(np.float64)
    if kind == "bf16":
        return np_bf16(w)
    if kind == "q4":
        return np_q4(w, scale)
    raise ValueError(kind)


def brute_force(layer: OracleLayer, x: np.ndarray) -> dict:
    """Evaluate all E experts on every token, then select, weight and join."""
    k = layer.w_kind
    X0 = x.astype(np.float64) if layer.x_kind == "f32" else np_bf16(x)       # [T,H]
    if layer.norm_w is not None:                                              # RMSNorm, then weight
        rho = 1.0 / np.sqrt(np.mean(X0 * X0, axis=1, keepdims=True) + layer.norm_eps)
        X = X0 * rho * layer.norm_w.astype(np.float64)
    else:
        X = X0
    Wg = np_decode(layer.gate, layer.gate_scale, k)                           # [E,I,H]
    Wu = np_decode(layer.up, layer.up_scale, k)
    Wd = np_decode(layer.down, layer.down_scale, k)                           # [E,H,I]
    G = np.einsum("eih,th->tei", Wg, X)
    U = np.einsum("eih,th->tei", Wu, X)
    A = G / (1.0 + np.exp(-G)) * U                                            # silu(g)*u
    Y = np.einsum("ehi,tei->teh", Wd, A)                                      # every expert [T,E,H]
    logits = X @ layer.router.astype(np.float64).T                            # [T,E]
    E = layer.n_experts
    order = np.lexsort((np.broadcast_to(np.arange(E), logits.shape), -logits), axis=-1)
    ids = order[:, :layer.top_k]
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(p, ids, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    routed = np.einsum("tj,tjh->th", w, np.take_along_axis(Y, ids[:, :, None], axis=1))
    Sg = X @ np_decode(layer.sh_gate, layer.sh_gate_scale, k).T
    Su = X @ np_decode(layer.sh_up, layer.sh_up_scale, k).T
    S = (Sg / (1.0 + np.exp(-Sg)) * Su) @ np_decode(layer.sh_down, layer.sh_down_scale, k).T
    s = 1.0 / (1.0 + np.exp(-(X @ layer.gate_vec.astype(np.float64))))
    out = routed + s[:, None] * S
    if layer.residual:
        out = X0 + out
    return {"out": out, "routed": routed, "shared": S, "gate": s, "ids": ids.astype(np.int32),
            "weights": w, "logits": logits, "all_experts": Y}
