"""Every workgroup barrier in the kernels waits for the wave's own LDS reads
and DMA first.

After a barrier another wave may issue global_load_lds into an LDS buffer
this wave was reading.  The workgroup fence of __syncthreads() orders LDS
accesses between waves, but not a read still in flight against such a DMA
write, and the compiler is free to schedule a read's consumer after the
barrier.  So in the gfx950 assembly of every kernel, each s_barrier must be
preceded -- after the last LDS access and the last VMEM load in the same
basic block -- by s_waitcnt with lgkmcnt(0) and vmcnt(0).  (A run-to-run
difference of one bf16 ulp in the forward pass came from exactly this: two
V-fragment reads still in flight at the barrier.)  CPU-only: hipcc emits the
assembly, no GPU is needed.
"""
import os
import re
import subprocess
import tempfile

import pytest

from exact_tiled_attention_30_amd import build

HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [build.hipcc(), *[f for f in build.compile_flags(src) if f != "-fPIC"],
           "--cuda-device-only", "-S", "-I", build.INCLUDE, "-I", build.CSRC,
           os.path.join(build.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read().split("\n")


def unguarded_barriers(lines):
    """(kernel, line) of each s_barrier lacking a full wait after the last
    LDS access / VMEM load before it in its basic block."""
    bad, kernel = [], None
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kernel = m.group(1)
        if "s_barrier" not in line:
            continue
        lgkm0 = vm0 = False
        for j in range(i - 1, -1, -1):
            t = lines[j].strip()
            if t.startswith(".LBB") or t.startswith("s_cbranch") or "s_barrier" in t or re.match(r"^_Z\w+:", t):
                break
            if t.startswith("s_waitcnt"):
                lgkm0 = lgkm0 or "lgkmcnt(0)" in t
                vm0 = vm0 or "vmcnt(0)" in t
            if t.startswith("ds_") and not lgkm0:
                bad.append((kernel, i + 1, "LDS access not waited"))
                break
            if (t.startswith("global_load") or t.startswith("buffer_load")) and not vm0:
                bad.append((kernel, i + 1, "VMEM load not waited"))
                break
    return bad


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_every_barrier_waits_for_lds_and_dma(src):
    with tempfile.TemporaryDirectory() as d:
        lines = _asm(src, d)
    # the MFMA yardstick has no LDS and no barrier; fa2_noalloc.hip holds no
    # kernel (only the static scratch and its entry point)
    if src not in ("fa2_calib.hip", "fa2_noalloc.hip"):
        assert any("s_barrier" in l for l in lines)
    assert unguarded_barriers(lines) == []
