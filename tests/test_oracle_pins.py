"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped scale, a
mask that is off by one or points the wrong way, a transposed operand, a wrong
[B, N, H, d] index, a missing normalisation, a wrong gradient term) fails at
least one of them.  None of them re-types the oracle's formula.

Definitions: infra-guide page "6.2 FlashAttention V2 in depth", section 5.1
(causal mask), section 6.1 (forward, saved logsumexp), section 7 (backward,
D vector); the FlashAttention-2 abstract (the result is exact).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _val(s):
    if isinstance(s, (int, float)):
        return float(s)
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    return float(Fraction(s))


def _bnhd(x):
    """[N, d] -> [1, N, 1, d]"""
    return np.asarray(x, np.float64)[None, :, None, :]


@pytest.mark.parametrize("name", ["hand_2x2.json", "hand_4x4.json"])
@pytest.mark.parametrize("mode", ["full", "causal"])
def test_golden_hand_cases(name, mode):
    case = json.load(open(os.path.join(GOLDEN, name)))
    scale = _val(case["scale"])
    o, lse = oracle.attention_forward(_bnhd(case["q"]), _bnhd(case["k"]), _bnhd(case["v"]),
                                      causal=(mode == "causal"), scale=scale)
    want_o = np.array([[_val(x) for x in row] for row in case[mode]["o"]])
    want_lse = np.array([_val(x) for x in case[mode]["lse"]])
    np.testing.assert_allclose(o[0, :, 0, :], want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], want_lse, rtol=0, atol=1e-14)


def _rand(B, N, H, d, scale=1.0):
    return RNG.standard_normal((B, N, H, d)) * scale


def _n_vis(N, causal):
    return np.arange(1, N + 1) if causal else np.full(N, N)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_softmax_sum_to_one(causal):
    # V = 1 everywhere: O_i = sum_j P_ij must be exactly 1 for every row.
    B, N, H, d = 2, 37, 3, 8
    q, k = _rand(B, N, H, d), _rand(B, N, H, d)
    v = np.ones((B, N, H, d))
    o, _ = oracle.attention_forward(q, k, v, causal, 0.7)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    B, N, H, d = 2, 29, 2, 6
    scale = 0.37
    q, v = _rand(B, N, H, d), _rand(B, N, H, d)
    kvec = RNG.standard_normal((H, d))
    k = np.broadcast_to(kvec[None, None], (B, N, H, d)).copy()
    o, lse = oracle.attention_forward(q, k, v, causal, scale)
    nv = _n_vis(N, causal)
    for b in range(B):
        for h in range(H):
            csum = np.cumsum(v[b, :, h, :], axis=0)
            mean = csum[nv - 1] / nv[:, None]
            np.testing.assert_allclose(o[b, :, h, :], mean, rtol=0, atol=1e-13)
            want = scale * (q[b, :, h, :] @ kvec[h]) + np.log(nv)
            np.testing.assert_allclose(lse[b, h], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_and_log_count(causal):
    B, N, H, d = 1, 23, 2, 5
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    o, lse = oracle.attention_forward(q, k, v, causal, 0.0)
    nv = _n_vis(N, causal)
    for h in range(H):
        mean = np.cumsum(v[0, :, h, :], axis=0)[nv - 1] / nv[:, None]
        np.testing.assert_allclose(o[0, :, h, :], mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], np.log(nv), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_dominant_score_returns_that_value_row(causal):
    # A large scale turns the softmax into a hard argmax over visible keys.
    B, N, H, d = 1, 40, 2, 8
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    scale = 1e4
    o, lse = oracle.attention_forward(q, k, v, causal, scale)
    nv = _n_vis(N, causal)
    checked = 0
    for h in range(H):
        for i in range(N):
            dots = k[0, : nv[i], h, :] @ q[0, i, h, :]
            order = np.sort(dots)
            if len(order) > 1 and scale * (order[-1] - order[-2]) < 60:
                continue  # runner-up not negligible; skip this row
            j = int(np.argmax(dots))
            np.testing.assert_allclose(o[0, i, h, :], v[0, j, h, :], rtol=0, atol=1e-12)
            assert abs(lse[0, h, i] - scale * dots[j]) <= 1e-9 * scale
            checked += 1
    assert checked > N  # most rows qualify


def test_joint_key_permutation_leaves_full_attention_unchanged():
    B, N, H, d = 2, 31, 3, 7
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    perm = RNG.permutation(N)
    o1, l1 = oracle.attention_forward(q, k, v, False, 0.5)
    o2, l2 = oracle.attention_forward(q, k[:, perm], v[:, perm], False, 0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_lse_only(causal):
    # k_j -> k_j + u adds scale*<q_i,u> to every score of row i: softmax is
    # unchanged and L_i moves by exactly that amount.
    B, N, H, d = 2, 26, 2, 5
    scale = 0.6
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    u = RNG.standard_normal((H, d))
    o1, l1 = oracle.attention_forward(q, k, v, causal, scale)
    o2, l2 = oracle.attention_forward(q, k + u[None, None], v, causal, scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    shift = scale * np.einsum("bnhd,hd->bhn", q, u)
    np.testing.assert_allclose(l2 - l1, shift, rtol=0, atol=1e-12)


def test_causal_special_rows_and_prefix_consistency():
    B, N, H, d = 2, 33, 2, 6
    scale = 0.45
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    oc, lc = oracle.attention_forward(q, k, v, True, scale)
    of, lf = oracle.attention_forward(q, k, v, False, scale)
    # row 0 sees only key 0
    np.testing.assert_allclose(oc[:, 0], v[:, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lc[:, :, 0], scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]),
                               rtol=0, atol=1e-14)
    # the last row sees every key, as without the mask
    np.testing.assert_allclose(oc[:, -1], of[:, -1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lc[:, :, -1], lf[:, :, -1], rtol=0, atol=1e-14)
    # rows < M do not depend on keys >= M
    M = 17
    om, lm = oracle.attention_forward(q[:, :M], k[:, :M], v[:, :M], True, scale)
    np.testing.assert_allclose(oc[:, :M], om, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lc[:, :, :M], lm, rtol=0, atol=1e-15)
    # and the mask is not reversed: the full and causal results differ elsewhere
    assert np.abs(oc[:, 1:-1] - of[:, 1:-1]).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds(causal):
    B, N, H, d = 1, 30, 2, 4
    scale = 0.8
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    _, lse = oracle.attention_forward(q, k, v, causal, scale)
    nv = _n_vis(N, causal)
    for h in range(H):
        for i in range(N):
            smax = scale * (k[0, : nv[i], h, :] @ q[0, i, h, :]).max()
            assert smax - 1e-12 <= lse[0, h, i] <= smax + math.log(nv[i]) + 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_heads_and_batches_are_independent(causal):
    # The [B, N, H, d] result for head (b, h) equals running that head alone.
    # Any slip in the layout index (e.g. treating the tensor as [B, H, N, d])
    # mixes heads or tokens and fails here.
    B, N, H, d = 3, 19, 4, 5
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    o, lse = oracle.attention_forward(q, k, v, causal, 0.9)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1), slice(None))
            o1, l1 = oracle.attention_forward(q[sl], k[sl], v[sl], causal, 0.9)
            np.testing.assert_array_equal(o[sl], o1)
            np.testing.assert_array_equal(lse[b, h], l1[0, 0])


def test_negative_scale_equals_negated_queries():
    B, N, H, d = 1, 21, 2, 6
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, causal, -0.3)
        o2, l2 = oracle.attention_forward(-q, k, v, causal, 0.3)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-15)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-15)


def test_selected_rows_match_full_result():
    B, N, H, d = 2, 25, 3, 4
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, causal, 0.5)
        rows = np.array([[0, 0, 0], [1, 2, 24], [1, 0, 13], [0, 1, 7]])
        orow, lrow = oracle.attention_forward_rows(q, k, v, causal, 0.5, rows)
        for r, (b, h, i) in enumerate(rows):
            np.testing.assert_array_equal(orow[r], o[b, i, h])
            assert lrow[r] == lse[b, h, i]


def test_bad_sizes_are_rejected():
    q = np.zeros((1, 4, 1, 2))
    with pytest.raises(RuntimeError):
        oracle.attention_forward_rows(q, q, q, False, 1.0, [[0, 0, 4]])
    with pytest.raises(RuntimeError):
        oracle.attention_backward(q, q, q, q, False, 1.0, heads=[[0, 1]])


# ---------------------------------------------------------------- backward --

def _objective(q, k, v, dout, causal, scale):
    o, _ = oracle.attention_forward(q, k, v, causal, scale)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    # Brute-force gradient of f(Q, K, V) = sum(dO * O) through the forward.
    B, N, H, d = 2, 5, 2, 3
    scale = 0.7
    q, k, v, dout = (_rand(B, N, H, d) for _ in range(4))
    g = oracle.attention_backward(q, k, v, dout, causal, scale)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name[1]] = xp
            args_m[name[1]] = xm
            fp = _objective(args_p["q"], args_p["k"], args_p["v"], dout, causal, scale)
            fm = _objective(args_m["q"], args_m["k"], args_m["v"], dout, causal, scale)
            num[idx] = (fp - fm) / (2 * eps)
        # oracle slabs are [B*H, N, d] in b-major head order
        got = g[name].reshape(B, H, N, d).transpose(0, 2, 1, 3)
        np.testing.assert_allclose(got, num, rtol=0, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_sums_and_D_identity(causal):
    B, N, H, d = 2, 24, 2, 6
    scale = 0.5
    q, k, v, dout = (_rand(B, N, H, d) for _ in range(4))
    g = oracle.attention_backward(q, k, v, dout, causal, scale)
    o, lse = oracle.attention_forward(q, k, v, causal, scale)
    dk = g["dk"].reshape(B, H, N, d)
    dv = g["dv"].reshape(B, H, N, d)
    # rows of dS sum to zero, so the key gradients sum to zero per head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    # rows of P sum to one, so the value gradients sum to the summed dO
    np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=1), rtol=0, atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals <dO_i, O_i> (section 7.3)
    np.testing.assert_allclose(g["D"].reshape(B, H, N),
                               np.einsum("bnhd,bnhd->bhn", dout, o), rtol=0, atol=1e-12)
    # the backward's own logsumexp is the forward's
    np.testing.assert_allclose(g["lse"].reshape(B, H, N), lse, rtol=0, atol=1e-13)


def test_backward_selected_heads_match_all_heads():
    B, N, H, d = 2, 9, 3, 4
    q, k, v, dout = (_rand(B, N, H, d) for _ in range(4))
    full = oracle.attention_backward(q, k, v, dout, True, 0.4)
    heads = [(1, 2), (0, 1)]
    part = oracle.attention_backward(q, k, v, dout, True, 0.4, heads=heads)
    for t, (b, h) in enumerate(heads):
        for name in ("dq", "dk", "dv", "lse", "D"):
            np.testing.assert_array_equal(part[name][t], full[name][b * H + h])
