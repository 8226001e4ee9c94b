"""Build libqlin.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python quantized_linear_layers_token_amd/build.py   (by path: importing the
package itself loads the library)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqlin.so")

ARCH = "gfx950"
SOURCES = ["quant_act.hip", "gemv.hip", "gemm_small.hip", "gemm_large.hip", "gemm_packed.hip", "linear.hip", "linear_tokens.hip", "weight_only.hip",
           "noalloc.hip",
           "qlin_api.hip"]
HEADERS = ["qlin_device.h", "qlin_internal.h", "qlin_round.h", "qlin_rows.h"]

# Never fast-math, never flush denormals: the quantizers are bit-exact against
# IEEE f32 divide / multiply / round-half-even.  Packed FP32 instructions are
# switched off for the device code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqlin.so)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), jobs: int = 0) -> str:
    """Compile every kernel source for gfx950 and link libqlin.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
