"""Build libfa2.so (the C-ABI HIP library) for gfx950 with hipcc.

Run as ``python -m exact_tiled_attention_30_amd.build`` or call ``build()``.
No GPU is needed: hipcc cross-compiles the gfx950 code object.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")

SOURCES = ["fa2_api.cpp", "fa2_dispatch.cpp", "fa2_fwd.hip", "fa2_bwd.hip", "fa2_fa1_order.hip", "fa2_calib.hip",
           "fa2_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 atomicAdd -> hardware global_atomic_add_f32 (device memory is coarse-grained)
    "-munsafe-fp-atomics",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile every HIP source into libfa2.so (always recompiles)."""
    out_tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv)
