"""Tolerance checks of library results against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark).

Forward (bf16 inputs, fp32 accumulation):
  * mean |dO| <= 1e-3 over all compared elements;
  * every element: |dO| <= 1e-2 + ulp_bf16(O_ref) / 2.  The half-ulp term is
    the rounding of the bf16 output itself; where |O_ref| >= 4 it exceeds
    1e-2, so the bare 1e-2 bound would fail even for exactly rounded results.
    The bare max |dO| is reported beside it;
  * max |dL| <= 1e-3 (absolute, natural-log logsumexp).
Gradients, per tensor G: max |dG| <= 5e-2 * max |G_ref| and
mean |dG| <= 5e-3 * mean |G_ref| (errors relative to the reference's own
magnitude).
"""
from __future__ import annotations

import numpy as np

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
G_MAX_REL = 5e-2
G_MEAN_REL = 5e-3


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, e - 8)


def _np(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, np.float64)


def forward_report(o, lse, o_ref, lse_ref) -> dict:
    o, lse, o_ref, lse_ref = _np(o), _np(lse), _np(o_ref), _np(lse_ref)
    do = np.abs(o - o_ref)
    excess = do - 0.5 * ulp_bf16(o_ref)
    dl = np.abs(lse - lse_ref)
    rep = {
        "max_abs_dO": float(do.max()) if do.size else 0.0,
        "mean_abs_dO": float(do.mean()) if do.size else 0.0,
        "max_dO_beyond_half_ulp": float(excess.max()) if do.size else 0.0,
        "max_abs_dLSE": float(dl.max()) if dl.size else 0.0,
        "all_finite": bool(np.isfinite(o).all() and np.isfinite(lse).all()),
    }
    rep["ok"] = bool(rep["all_finite"]
                     and rep["mean_abs_dO"] <= O_MEAN_ABS
                     and rep["max_dO_beyond_half_ulp"] <= O_MAX_ABS
                     and rep["max_abs_dLSE"] <= LSE_MAX_ABS)
    return rep


def gradient_report(g, g_ref) -> dict:
    g, g_ref = _np(g), _np(g_ref)
    d = np.abs(g - g_ref)
    ref_max = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    ref_mean = float(np.abs(g_ref).mean()) if g_ref.size else 0.0
    rep = {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "ref_max": ref_max,
        "ref_mean": ref_mean,
        "all_finite": bool(np.isfinite(g).all()),
    }
    rep["max_rel"] = rep["max_abs"] / ref_max if ref_max > 0 else rep["max_abs"]
    rep["mean_rel"] = rep["mean_abs"] / ref_mean if ref_mean > 0 else rep["mean_abs"]
    rep["ok"] = bool(rep["all_finite"] and rep["max_rel"] <= G_MAX_REL
                     and rep["mean_rel"] <= G_MEAN_REL)
    return rep
