"""Builds libmoe_ffn.so for gfx950 in-tree (moe_decode_ffn_amd/lib/), and the
layer_loop driver (a C-ABI-only program for profiler runs) beside it.

    python -m moe_decode_ffn_amd.build [--changed]

Every HIP source is compiled with hipcc for gfx950 only, with packed fp32
instructions disabled (-packed-fp32-ops) and no floating-point contraction
(the kernels spell out every fused multiply-add they want, so results do
not depend on the compiler's contraction choices).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBRARY = os.path.join(LIBDIR, "libmoe_ffn.so")
DRIVER_SRC = os.path.join(PKG, "driver", "layer_loop.hip")
DRIVER = os.path.join(LIBDIR, "layer_loop")
OBJDIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}"]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _up_to_date(src: str, obj: str) -> bool:
    """The object is newer than its source and every header it may include."""
    if not os.path.exists(obj):
        return False
    deps = [src] + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(INCLUDE, "moe_ffn.h"))
    return all(os.path.getmtime(obj) > os.path.getmtime(d) for d in deps)


def _compile(src: str, force: bool = True) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    if not force and _up_to_date(src, obj):
        return obj
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build_library(jobs: int | None = None, force: bool = True) -> str:
    """Compiles every source (force=False: only those whose object is out of date) and
    links the library."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, force), srcs))
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    return LIBRARY


def build_driver() -> str:
    """layer_loop, linked against the in-tree library (found next to it at run time)."""
    tmp = DRIVER + ".tmp"
    cmd = [HIPCC, *COMMON, DRIVER_SRC, "-o", tmp, f"-L{LIBDIR}", "-lmoe_ffn", "-Wl,-rpath,$ORIGIN"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {DRIVER_SRC}:\n{r.stderr}")
    os.replace(tmp, DRIVER)
    return DRIVER


if __name__ == "__main__":
    print(build_library(force="--changed" not in sys.argv))
    print(build_driver())
    sys.exit(0)
