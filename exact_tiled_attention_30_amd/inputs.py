"""Seeded synthetic attention inputs shared by the tests, the benchmark and the
smoke check.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to bfloat16.  Both the HIP library and the fp64 reference receive
exactly the tensors made here.

Recipe (one fresh CPU generator per workload, seeded with `seed`):
  1. draw float32 standard normals in the order Q, K, V, each [B, N, H, d];
  2. if `peaked_fraction` > 0, draw a permutation of the B*N*H key rows and
     take the first round(peaked_fraction * B*N*H) of them;
  3. if `with_dout`, draw dO the same way;
  4. round every tensor to bfloat16 (round to nearest even), then multiply the
     chosen key rows by 8 (exact: a power of two) to create peaked softmax rows.

The shapes follow the attention workloads the FlashAttention-2 pages measure
(sequence lengths 1K-16K and beyond, head dim 64 and 128, causal and not).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, masking and the input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    peaked_fraction: float = 0.0
    backward: bool = False
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Forward FLOPs by the usual convention: 4*B*H*N^2*d, halved if causal;
        a backward pass is counted as 2.5x its forward."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        if self.causal:
            f *= 0.5
        return f * 2.5 if self.backward else f


def make_inputs(B: int, H: int, N: int, d: int, seed: int = 0,
                peaked_fraction: float = 0.0, with_dout: bool = False):
    """Return a dict of bfloat16 CPU tensors q, k, v (and dout) of shape [B, N, H, d]."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (B, N, H, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    rows = None
    n_rows = B * N * H
    if peaked_fraction > 0.0 and n_rows > 0:
        n_pick = int(round(peaked_fraction * n_rows))
        rows = torch.randperm(n_rows, generator=g)[:n_pick]
    dout = torch.randn(shape, generator=g, dtype=torch.float32) if with_dout else None
    out = {
        "q": q.to(torch.bfloat16),
        "k": k.to(torch.bfloat16),
        "v": v.to(torch.bfloat16),
    }
    if rows is not None and rows.numel() > 0:
        kr = out["k"].view(n_rows, d)
        kr[rows] = kr[rows] * 8
    if dout is not None:
        out["dout"] = dout.to(torch.bfloat16)
    return out


def make_inputs_on_device(B: int, H: int, N: int, d: int, seed: int = 0,
                          with_dout: bool = False, device: str = "cuda"):
    """The same recipe as make_inputs -- N(0,1) fp32 draws rounded to bf16, in
    the order q, k, v (, dout) -- but drawn by torch's generator on the device,
    one batch entry at a time, for tensors too large to draw on the host.  The
    values differ from make_inputs' for the same seed (another generator)."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = {}
    for name in ("q", "k", "v") + (("dout",) if with_dout else ()):
        t = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=device)
        for b in range(B):
            t[b] = torch.randn((N, H, d), generator=g, dtype=torch.float32,
                               device=device).to(torch.bfloat16)
        out[name] = t
    return out


def workload(name: str) -> Workload:
    """A named workload, or one spelled fwd_b{B}_h{H}_n{N}_d{d}_{full|causal}
    (or bwd_...) with the default recipe (seed 0, no peaked rows)."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    import re

    m = re.fullmatch(r"(fwd|bwd)_b(\d+)_h(\d+)_n(\d+)_d(\d+)_(full|causal)", name)
    if not m:
        raise KeyError(f"unknown workload {name!r}")
    kind, B, H, N, d, mask = m.groups()
    return Workload(name, int(B), int(H), int(N), int(d), mask == "causal",
                    backward=kind == "bwd")


def inputs_for(w: Workload):
    return make_inputs(w.B, w.H, w.N, w.d, seed=w.seed,
                       peaked_fraction=w.peaked_fraction, with_dout=w.backward)


def _sweep():
    out = []
    for N in (2048, 4096, 8192, 16384):
        B = 16384 // N
        for d, H in ((64, 32), (128, 16)):
            for causal in (False, True):
                tag = "causal" if causal else "full"
                out.append(Workload(f"fwd_b{B}_h{H}_n{N}_d{d}_{tag}", B, H, N, d, causal))
    return out


# The measured workloads.  Names state what each one is.
WORKLOADS = {w.name: w for w in [
    Workload("fwd_b1_h1_n128_d64_full", 1, 1, 128, 64, False),
    Workload("fwd_b8_h16_n1024_d64_full", 8, 16, 1024, 64, False),
    Workload("fwd_b8_h16_n1024_d64_causal", 8, 16, 1024, 64, True),
    *_sweep(),
    Workload("fwd_b1_h16_n32768_d128_causal_peaked", 1, 16, 32768, 128, True,
             peaked_fraction=0.01),
    Workload("bwd_b4_h16_n4096_d128_causal", 4, 16, 4096, 128, True, backward=True),
    # few heads, long sequence: B*H*ceil(N/256) = 128 workgroups cannot fill
    # 256 CUs (the case split-KV is for)
    Workload("fwd_b1_h2_n16384_d128_full", 1, 2, 16384, 128, False),
]}
