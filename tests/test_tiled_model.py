"""A tiled fp64 model of the FlashAttention-2 forward, checked against the
plain-definition oracle (CPU only).

The model follows the algorithm of infra-guide page "6.2 FlashAttention V2 in
depth", section 6.1, in fp64 and written from its description: an outer loop
over Q tiles of B_r rows, an inner loop over K/V tiles of B_c keys, a running
row max m and row sum l, an unnormalised O that is rescaled by exp(m_old -
m_new) when the max moves, one division by l after the key loop, and
L = m + log(l) saved for the backward.  For the causal case (section 5.3) the
key loop of a Q tile starting at row i stops at min(N, i + B_r), and a K/V
tile is masked element by element only when it reaches past the tile's first
row.  Equality with the naive oracle to about 1e-12 pins that algebra (the
delayed normalisation is exact, per the FlashAttention-2 abstract) and those
two bounds independently of the GPU.  A second test checks the causal tile
classification (skip / whole / diagonal) against the element mask by brute
force.
"""
import numpy as np
import pytest

import oracle


def tile_class(i0, br, j0, bc, n):
    """Causal classification of K/V tile [j0, j0+bc) for Q tile [i0, i0+br),
    from the tile bounds alone: 'skip' if no row of the Q tile sees any of its
    keys, 'whole' if every row sees every key, else 'diagonal'."""
    last_row = min(i0 + br, n) - 1
    last_key = min(j0 + bc, n) - 1
    if j0 > last_row:
        return "skip"
    if last_key <= i0:
        return "whole"
    return "diagonal"


def tiled_forward(q, k, v, causal, scale, br, bc):
    """q, k, v: fp64 [N, d] of one head.  Returns (o [N, d], lse [N])."""
    n, d = q.shape
    o = np.zeros((n, d))
    lse = np.zeros(n)
    for i0 in range(0, n, br):
        rows = slice(i0, min(i0 + br, n))
        qi = q[rows]
        nr = qi.shape[0]
        m = np.full(nr, -np.inf)
        l = np.zeros(nr)
        acc = np.zeros((nr, d))
        kv_end = min(n, i0 + br) if causal else n
        for j0 in range(0, kv_end, bc):
            cols = slice(j0, min(j0 + bc, kv_end))
            s = scale * (qi @ k[cols].T)
            if causal and tile_class(i0, br, j0, bc, n) == "diagonal":
                r = np.arange(i0, i0 + nr)[:, None]
                c = np.arange(j0, j0 + s.shape[1])[None, :]
                s = np.where(c <= r, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        o[rows] = acc / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


CASES = [(1, 64, 64), (37, 16, 16), (130, 64, 32), (200, 32, 64), (257, 128, 64), (96, 48, 40)]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("n,br,bc", CASES)
def test_tiled_model_equals_naive_attention(n, br, bc, causal):
    rng = np.random.default_rng(n * 1000 + br + bc)
    d = 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    k[rng.integers(n)] *= 6.0  # one dominant key: the running max moves
    scale = 0.7
    o_t, l_t = tiled_forward(q, k, v, causal, scale, br, bc)
    o_n, l_n = oracle.attention_forward(q[None, :, None, :], k[None, :, None, :],
                                        v[None, :, None, :], causal, scale)
    assert np.abs(o_t - o_n[0, :, 0, :]).max() < 1e-12
    assert np.abs(l_t - l_n[0, 0]).max() < 1e-12


@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 256, 333])
@pytest.mark.parametrize("br,bc", [(32, 32), (128, 64), (256, 64), (64, 128), (48, 80)])
def test_causal_tile_classes_match_the_element_mask(n, br, bc):
    for i0 in range(0, n, br):
        rows = np.arange(i0, min(i0 + br, n))
        for j0 in range(0, n, bc):
            keys = np.arange(j0, min(j0 + bc, n))
            visible = keys[None, :] <= rows[:, None]
            want = "skip" if not visible.any() else ("whole" if visible.all() else "diagonal")
            assert tile_class(i0, br, j0, bc, n) == want, (n, br, bc, i0, j0)
            # the key loop's bound: a Q tile never needs keys at or past i0 + br
            if j0 >= min(n, i0 + br):
                assert want == "skip"
