"""Pins of the parity checker (oracle/compare.py) itself.

Every GPU parity test ends in forward_report or gradient_report, so a slip
that loosened them would let wrong results through unnoticed.  These CPU
tests fix the checker to its stated bounds:

  * ulp_bf16 equals the spacing of bfloat16 numbers that torch's own
    bfloat16 nextafter gives, for every finite bfloat16 value (zero and the
    subnormals included), and bounds the round-to-nearest error of torch's
    fp32 -> bf16 conversion, with equality half-way between two values;
  * each bound -- mean |dO| <= 1e-3, |dO| <= 1e-2 + ulp/2 per element,
    |dL| <= 1e-3, max |dG| <= 5e-2 max |G_ref|, mean |dG| <= 5e-3 mean |G_ref|
    -- accepts a result 1e-9 (relative) inside it and rejects one 1e-9 past
    it, with errors of either sign, in several bf16 binades;
  * NaN and infinity are rejected; errors against an all-zero reference are
    held to the same bounds in absolute terms;
  * a gradient reference below bf16's normal range is met by the exactly
    rounded result and missed by one 3/4 of a bf16 spacing off;
  * planted slips in a copy of the checker's source -- any bound loosened by
    1 %, the ulp term doubled or dropped to the old zero-spacing form, an
    absolute value dropped, the subnormal floor widened or applied to
    normal-range elements -- each make one of these pins fail.
"""
import os
import types

import numpy as np
import pytest
import torch

from oracle import compare

EPS = 1e-9
IN, PAST = 1.0 - EPS, 1.0 + EPS
BINADES = [0.0, 0.3, -0.7, 1.5, 6.0, -6.0, 40.0]
N_EL = 4000  # one large error among N_EL elements keeps the mean far below 1e-3

# The bounds as stated; the cases below are built from these numbers, not
# from the module under test, so a loosened module cannot move them.
O_MAX, O_MEAN, LSE_MAX, G_MAX, G_MEAN = 1e-2, 1e-3, 1e-3, 5e-2, 5e-3


def bf16_spacing(v):
    """Spacing of bf16 numbers at |v| from torch's bf16 nextafter."""
    x = torch.tensor([abs(v)], dtype=torch.float64).to(torch.bfloat16)
    if float(x) > abs(v):  # rounded up into the next binade: step back
        x = torch.nextafter(x, torch.zeros_like(x))
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    return float(up.double() - x.double())


# ---- cases -------------------------------------------------------------------

def fwd_arrays(o_ref_val, d_el=0.0, d_all=0.0, d_lse=0.0, sign=1.0):
    o_ref = np.full(N_EL, o_ref_val, np.float64)
    o = o_ref + sign * d_all
    if d_el:
        o[7] = o_ref[7] + sign * d_el
    lse_ref = np.linspace(-3.0, 12.0, 64)
    lse = lse_ref.copy()
    lse[5] += sign * d_lse
    return o, lse, o_ref, lse_ref


def element_bound(v):
    return O_MAX + 0.5 * bf16_spacing(v)


def forward_cases(factor):
    cases = []
    for v in BINADES:
        for s in (1.0, -1.0):
            cases.append(fwd_arrays(v, d_el=element_bound(v) * factor, sign=s))
    for s in (1.0, -1.0):
        cases.append(fwd_arrays(0.3, d_all=O_MEAN * factor, sign=s))
        cases.append(fwd_arrays(0.3, d_lse=LSE_MAX * factor, sign=s))
    return cases


def grad_arrays(d_max_rel=0.0, d_mean_rel=0.0, sign=1.0):
    ref = np.random.default_rng(1).standard_normal((3, 257, 64))
    g = ref + sign * d_mean_rel * np.abs(ref).mean()
    if d_max_rel:
        g[1, 100, 5] = ref[1, 100, 5] + sign * d_max_rel * np.abs(ref).max()
    return g, ref


def gradient_cases(factor):
    cases = []
    for s in (1.0, -1.0):
        cases.append(grad_arrays(d_max_rel=G_MAX * factor, sign=s))
        cases.append(grad_arrays(d_mean_rel=G_MEAN * factor, sign=s))
    return cases


# ---- the pins, written against a checker module `m` ---------------------------

def pin_ulp_matches_nextafter(m):
    bits = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16)  # +0 .. max finite
    x = bits.view(torch.bfloat16)[:-1]  # the largest finite value has no finite successor
    up = torch.nextafter(x, torch.full_like(x, float("inf")))
    spacing = (up.double() - x.double()).numpy()
    assert np.array_equal(m.ulp_bf16(x.double().numpy()), spacing)
    assert np.array_equal(m.ulp_bf16(-x.double().numpy()), spacing)


def pin_half_ulp_bounds_rounding(m):
    g = torch.Generator().manual_seed(0)
    n = 200000
    x = torch.randn(n, generator=g) * torch.exp2(
        torch.randint(-140, 20, (n,), generator=g).float())
    err = (x.to(torch.bfloat16).double() - x.double()).abs().numpy()
    assert (err <= 0.5 * m.ulp_bf16(x.double().numpy())).all()
    mid = torch.tensor([1.0 + 2.0 ** -8, 3.0 + 2.0 ** -7, 2.0 ** -130 + 2.0 ** -134])
    err_mid = (mid.to(torch.bfloat16).double() - mid.double()).abs().numpy()
    assert np.array_equal(err_mid, 0.5 * m.ulp_bf16(mid.double().numpy()))


def pin_forward_bounds(m):
    for args in forward_cases(IN):
        rep = m.forward_report(*args)
        assert rep["ok"], rep
    for args in forward_cases(PAST):
        rep = m.forward_report(*args)
        assert not rep["ok"], rep


def pin_forward_non_finite(m):
    for bad in (np.nan, np.inf, -np.inf):
        o_ref = np.zeros(16)
        o = o_ref.copy()
        o[3] = bad
        assert not m.forward_report(o, np.zeros(4), o_ref, np.zeros(4))["ok"]
        lse = np.zeros(4)
        lse[1] = bad
        assert not m.forward_report(o_ref, lse, o_ref, np.zeros(4))["ok"]


def pin_forward_literal_bound_reported(m):
    # an element at |O| = 6 may miss by 1e-2 plus half its bf16 spacing:
    # accepted, but reported as over the bare 1e-2
    rep = m.forward_report(*fwd_arrays(6.0, d_el=0.02))
    assert rep["ok"] and not rep["max_abs_dO_le_1e-2"]
    assert rep["max_abs_dO"] == pytest.approx(0.02)
    rep = m.forward_report(*fwd_arrays(6.0, d_el=0.0099))
    assert rep["ok"] and rep["max_abs_dO_le_1e-2"]


def pin_gradient_bounds(m):
    for args in gradient_cases(IN):
        rep = m.gradient_report(*args)
        assert rep["ok"], rep
    for args in gradient_cases(PAST):
        rep = m.gradient_report(*args)
        assert not rep["ok"], rep


def pin_gradient_non_finite_and_zero_reference(m):
    g, ref = grad_arrays()
    g[0, 0, 0] = np.nan
    assert not m.gradient_report(g, ref)["ok"]
    # an all-zero reference: absolute errors against the same bounds
    z = np.zeros((2, 8, 64))
    assert m.gradient_report(z, z)["ok"]
    noise = z + 1e-7
    assert m.gradient_report(noise, z)["ok"]
    one = z.copy()
    one[1, 2, 3] = G_MAX * PAST
    assert not m.gradient_report(one, z)["ok"]
    assert not m.gradient_report(z + G_MEAN * PAST, z)["ok"]


def pin_gradient_subnormal_reference(m):
    # a reference below bf16's normal range: the exactly rounded result passes,
    # one off by three quarters of a bf16 spacing (2^-133) everywhere does
    # not, and normal-range elements of the same tensor keep the stated rule
    ref = np.random.default_rng(3).standard_normal((2, 64, 64)) * 1e-39
    rounded = torch.from_numpy(ref).float().to(torch.bfloat16).double().numpy()
    assert m.gradient_report(rounded, ref)["ok"]
    assert not m.gradient_report(ref + 0.75 * 2.0 ** -133, ref)["ok"]
    mixed = ref.copy()
    mixed[0] = np.random.default_rng(4).standard_normal((64, 64))
    g = mixed.copy()
    g[0] += G_MEAN * np.abs(mixed).mean() * 2 * PAST  # the normal half alone past the mean bound
    assert not m.gradient_report(g, mixed)["ok"]


PINS = [pin_ulp_matches_nextafter, pin_half_ulp_bounds_rounding, pin_forward_bounds,
        pin_forward_non_finite, pin_forward_literal_bound_reported, pin_gradient_bounds,
        pin_gradient_non_finite_and_zero_reference, pin_gradient_subnormal_reference]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_checker_pin(pin):
    pin(compare)


def test_stated_bounds_are_the_checkers():
    assert (compare.O_MAX_ABS, compare.O_MEAN_ABS, compare.LSE_MAX_ABS, compare.G_MAX_REL,
            compare.G_MEAN_REL) == (O_MAX, O_MEAN, LSE_MAX, G_MAX, G_MEAN)


# ---- planted slips -------------------------------------------------------------

SRC = open(os.path.join(os.path.dirname(compare.__file__), "compare.py")).read()

MUTANTS = {
    "loose_element_bound": ("O_MAX_ABS = 1e-2", "O_MAX_ABS = 1.01e-2"),
    "loose_mean_bound": ("O_MEAN_ABS = 1e-3", "O_MEAN_ABS = 1.01e-3"),
    "loose_lse_bound": ("LSE_MAX_ABS = 1e-3", "LSE_MAX_ABS = 1.01e-3"),
    "loose_grad_max": ("G_MAX_REL = 5e-2", "G_MAX_REL = 5.05e-2"),
    "loose_grad_mean": ("G_MEAN_REL = 5e-3", "G_MEAN_REL = 5.05e-3"),
    "full_ulp_term": ("excess = do - 0.5 * ulp_bf16(o_ref)", "excess = do - ulp_bf16(o_ref)"),
    "ulp_one_binade_up": ("np.maximum(e - 8, _BF16_MIN_EXP)", "np.maximum(e - 7, _BF16_MIN_EXP)"),
    "ulp_at_zero_from_frexp": (
        "e = np.where(a == 0.0, _BF16_MIN_EXP, np.maximum(e - 8, _BF16_MIN_EXP))",
        "e = e - 8"),
    "signed_output_error": ("do = np.abs(o - o_ref)", "do = o - o_ref"),
    "signed_lse_error": ("dl = np.abs(lse - lse_ref)", "dl = lse - lse_ref"),
    "signed_gradient_error": ("d = np.abs(g - g_ref)", "d = g - g_ref"),
    "floor_everywhere": ("sub = np.abs(g_ref) < 2.0 ** -126", "sub = np.abs(g_ref) >= 0"),
    "full_spacing_floor": ("np.maximum(d - 0.5 * ulp_bf16(g_ref), 0.0)",
                           "np.maximum(d - ulp_bf16(g_ref), 0.0)"),
}


def mutant_module(name):
    before, after = MUTANTS[name]
    assert SRC.count(before) == 1, f"mutation site for {name} not found"
    mod = types.ModuleType(f"compare_{name}")
    exec(compile(SRC.replace(before, after), f"<compare {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_slip_is_caught(name):
    m = mutant_module(name)
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted slip {name}"
