"""Tolerance checks of library results against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark).

Forward (bf16 inputs, fp32 accumulation):
  * mean |dO| <= 1e-3 over all compared elements;
  * every element: |dO| <= 1e-2 + ulp_bf16(O_ref) / 2.  The half-ulp term is
    the rounding of the bf16 output itself; where |O_ref| >= 4 it exceeds
    1e-2, so the bare 1e-2 bound would fail even for exactly rounded results.
    The bare max |dO| and its verdict against 1e-2 are reported beside it
    ("max_abs_dO", "max_abs_dO_le_1e-2"); only the ulp-aware rule decides "ok";
  * max |dL| <= 1e-3 (absolute, natural-log logsumexp).
Gradients, per tensor G: max |dG| <= 5e-2 * max |G_ref| and
mean |dG| <= 5e-3 * mean |G_ref| (errors relative to the reference's own
magnitude).  Where an element of G_ref lies below bf16's normal range
(|G_ref| < 2^-126, which takes a scale below about 1e-38 for dQ and dK), no
bf16 result can come closer than its own rounding, whose spacing there is a
fixed 2^-133: such an element's error counts only beyond half that spacing,
as in the forward's per-element rule.  Elements in the normal range are
compared exactly as stated.

Every comparison is "<=": a result exactly at a bound passes, one a rounding
step past it fails (pinned by tests/test_compare_pins.py).  Any NaN or
infinity in a result fails.
"""
from __future__ import annotations

import numpy as np

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
G_MAX_REL = 5e-2
G_MEAN_REL = 5e-3

# bfloat16 keeps fp32's exponent range with 8 significant bits: in the binade
# [2^(e-1), 2^e) its spacing is 2^(e-8); below the smallest normal, 2^-126,
# the subnormals are evenly spaced by 2^-133 (also the spacing at 0).
_BF16_MIN_EXP = -133


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x|: 2^(e-8) for |x| in [2^(e-1), 2^e),
    2^-133 for |x| below the smallest normal (2^-126), zero included."""
    a = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(a)
    e = np.where(a == 0.0, _BF16_MIN_EXP, np.maximum(e - 8, _BF16_MIN_EXP))
    return np.ldexp(1.0, e)


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
    finite = bool(np.isfinite(o).all() and np.isfinite(lse).all())
    rep = {
        "max_abs_dO": float(do.max()) if do.size else 0.0,
        "mean_abs_dO": float(do.mean()) if do.size else 0.0,
        "max_dO_beyond_half_ulp": float(excess.max()) if do.size else 0.0,
        "max_abs_dLSE": float(dl.max()) if dl.size else 0.0,
        "all_finite": finite,
    }
    # the literal reading, reported only (see the module docstring)
    rep["max_abs_dO_le_1e-2"] = bool(finite and rep["max_abs_dO"] <= O_MAX_ABS)
    rep["ok"] = bool(finite
                     and rep["mean_abs_dO"] <= O_MEAN_ABS
                     and rep["max_dO_beyond_half_ulp"] <= O_MAX_ABS
                     and rep["max_abs_dLSE"] <= LSE_MAX_ABS)
    return rep


def gradient_report(g, g_ref) -> dict:
    g, g_ref = _np(g), _np(g_ref)
    d = np.abs(g - g_ref)
    sub = np.abs(g_ref) < 2.0 ** -126
    if sub.any():
        d = np.where(sub, np.maximum(d - 0.5 * ulp_bf16(g_ref), 0.0), d)
    ref_max = float(np.abs(g_ref).max()) if g_ref.size else 0.0
    ref_mean = float(np.abs(g_ref).mean()) if g_ref.size else 0.0
    rep = {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "ref_max": ref_max,
        "ref_mean": ref_mean,
        "all_finite": bool(np.isfinite(g).all()),
    }
    # An all-zero reference (dQ and dK of a single visible key, where
    # dS = P (dP - D) vanishes; any gradient at scale = 0) has no magnitude of
    # its own: its errors are compared in absolute terms against the same
    # numbers, so the fp32 rounding noise of dP - D passes and O(1) errors
    # do not.
    rep["max_rel"] = rep["max_abs"] / ref_max if ref_max > 0 else rep["max_abs"]
    rep["mean_rel"] = rep["mean_abs"] / ref_mean if ref_mean > 0 else rep["mean_abs"]
    rep["ok"] = bool(rep["all_finite"] and rep["max_rel"] <= G_MAX_REL
                     and rep["mean_rel"] <= G_MEAN_REL)
    return rep
