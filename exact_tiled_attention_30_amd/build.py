"""Build libfa2.so (the C-ABI HIP library) for gfx950 with hipcc.

Run as ``python -m exact_tiled_attention_30_amd.build`` or call ``build()``.
No GPU is needed: hipcc cross-compiles the gfx950 code object.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")

SOURCES = ["fa2_api.cpp", "fa2_dispatch.cpp", "fa2_fwd.hip", "fa2_fwd_wide.hip", "fa2_bwd.hip",
           "fa2_fa1_order.hip", "fa2_calib.hip", "fa2_noalloc.hip"]

# Flags of one source only.  The 8-wave d = 128 forward kernels are built with
# LLVM's ILP-first machine scheduler, which measured faster for them alone.
SOURCE_FLAGS = {
    "fa2_fwd_wide.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}

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


def compile_flags(source: str) -> list:
    """hipcc flags of one translation unit (without -shared)."""
    return [f for f in HIPCC_FLAGS if f != "-shared"] + SOURCE_FLAGS.get(source, [])


def build(verbose: bool = False, resource_usage: bool = False, csrc: str = CSRC,
          out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every source (always recompiles, in parallel) and link libfa2.so."""
    with tempfile.TemporaryDirectory() as tmp:
        cmds = []
        for s in SOURCES:
            cmd = [hipcc(), *compile_flags(s), *extra_flags, "-I", INCLUDE, "-I", csrc]
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
            cmds.append(cmd + ["-c", os.path.join(csrc, s), "-o", os.path.join(tmp, s + ".o")])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        quiet = not (verbose or resource_usage)
        with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
            runs = list(ex.map(lambda c: subprocess.run(c, capture_output=quiet, text=True), cmds))
        for c, r in zip(cmds, runs):
            if r.returncode != 0:
                if quiet:
                    sys.stderr.write(r.stdout + r.stderr)
                raise subprocess.CalledProcessError(r.returncode, c)
        out_tmp = out + ".tmp"
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
                *[c[-1] for c in cmds], "-o", out_tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv)
