"""Properties of attention with a closed form at any size, checked on the GPU
at the full workload sizes (every element, no oracle run needed):

  * V = ones: every row of the softmax sums to 1, so O = 1 and, on random Q
    and K, the kernels' row sums, rescales and 1/l are exercised end to end.
  * All keys of a head equal: every visible score of a row is the same, so P is
    uniform, O_i is the mean of the visible V rows (a prefix mean when causal)
    and L_i = scale * q_i.k + ln(n_visible).
  * Backward: rows of dS sum to 0, so sum_j dK_j = 0; rows of P sum to 1, so
    sum_j dV_j = sum_i dO_i.
  * Causal row 0 sees only key 0 (O_0 = V_0 exactly); the causal last row
    sees every key (it equals the non-causal one); causal rows below M do not
    depend on the tokens at or past M (prefix consistency); without a mask,
    permuting the keys and values together changes nothing.  These compare
    two GPU results, each within rounding of the exact value.

Expected values are computed in fp64 on the host from the same bf16 inputs;
the forward comparison uses the forward tolerance (oracle/compare.py).
"""
import numpy as np
import pytest
import torch

from exact_tiled_attention_30_amd import binding
from exact_tiled_attention_30_amd.inputs import make_inputs
from oracle.compare import forward_report

pytestmark = pytest.mark.gpu

SHAPES = [(8, 16, 1024, 64), (1, 16, 16384, 128), (2, 32, 8192, 64)]
IDS = ["b8h16n1024d64", "b1h16n16384d128", "b2h32n8192d64"]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_ones_values_give_ones(shape, causal):
    B, H, N, d = shape
    print(f"[prop ones] {shape} causal={causal}", flush=True)
    x = make_inputs(B, H, N, d, seed=31)
    q, k = x["q"].cuda(), x["k"].cuda()
    v = torch.ones_like(q)
    o, lse = binding.attention_forward(q, k, v, causal, d ** -0.5)
    torch.cuda.synchronize()
    err = (o.float() - 1.0).abs().max().item()
    # O = sum_j bf16(P_j) / sum_j P_j, then rounded to bf16: within the
    # relative rounding of P (2^-9) and half a bf16 ulp at 1 (2^-8)
    assert err <= 2.0 ** -9 + 2.0 ** -8, err
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_identical_keys_give_prefix_means(shape, causal):
    B, H, N, d = shape
    scale = d ** -0.5
    print(f"[prop keys] {shape} causal={causal}", flush=True)
    x = make_inputs(B, H, N, d, seed=37)
    k = x["k"][:, :1].expand(B, N, H, d).contiguous()  # key 0 of each head, repeated
    o, lse = binding.attention_forward(x["q"].cuda(), k.cuda(), x["v"].cuda(), causal, scale)
    torch.cuda.synchronize()
    v64 = x["v"].double()
    n_vis = torch.arange(1, N + 1, dtype=torch.float64) if causal else torch.full((N,), float(N),
                                                                                   dtype=torch.float64)
    if causal:
        o_ref = v64.cumsum(dim=1) / n_vis.view(1, N, 1, 1)
    else:
        o_ref = v64.mean(dim=1, keepdim=True).expand(B, N, H, d)
    qk = (x["q"].double() * k.double()).sum(-1)              # [B, N, H]
    lse_ref = (scale * qk).permute(0, 2, 1) + torch.log(n_vis).view(1, 1, N)
    rep = forward_report(o.cpu(), lse.cpu(), o_ref.numpy(), lse_ref.numpy())
    print(f"  {rep}", flush=True)
    assert rep["ok"], rep


@pytest.mark.parametrize("atomic_dq", [False, True], ids=["two_pass", "atomic_dq"])
def test_gradient_sums_at_full_size(atomic_dq):
    B, H, N, d = 4, 16, 4096, 128
    print(f"[prop grad sums] B{B} H{H} N{N} d{d} causal atomic_dq={atomic_dq}", flush=True)
    x = {n: t.cuda() for n, t in make_inputs(B, H, N, d, seed=41, with_dout=True).items()}
    o, lse = binding.attention_forward(x["q"], x["k"], x["v"], True, d ** -0.5)
    dq, dk, dv = binding.attention_backward(x["q"], x["k"], x["v"], o, lse, x["dout"], True,
                                            d ** -0.5, atomic_dq=atomic_dq)
    torch.cuda.synchronize()
    dk, dv, do = dk.double(), dv.double(), x["dout"].double()
    sk = dk.sum(dim=1).abs() / dk.abs().sum(dim=1)
    sv = (dv.sum(dim=1) - do.sum(dim=1)).abs() / do.abs().sum(dim=1)
    print(f"  max |sum dK| / sum |dK| = {sk.max().item():.2e}, "
          f"max |sum dV - sum dO| / sum |dO| = {sv.max().item():.2e}", flush=True)
    assert sk.max().item() <= 1e-2
    assert sv.max().item() <= 1e-2
    assert np.isfinite(dq.float().cpu().numpy()).all()


def _close(a, b, what):
    """Two GPU results of the same rows: each is within rounding of the exact
    value, so they agree to the forward tolerance (1e-2 absolute plus a bf16
    ulp for large values)."""
    a, b = a.double(), b.double()
    tol = 1e-2 + 2.0 ** -7 * b.abs()
    bad = ((a - b).abs() > tol).sum().item()
    assert bad == 0, (what, bad, (a - b).abs().max().item())


@pytest.mark.parametrize("shape", SHAPES[:2], ids=IDS[:2])
def test_causal_first_and_last_rows(shape):
    # row 0 sees only key 0: O_0 = V_0 exactly, L_0 = scale * q_0.k_0; the
    # last row sees every key: it equals the non-causal last row
    B, H, N, d = shape
    scale = d ** -0.5
    x = {n: t.cuda() for n, t in make_inputs(B, H, N, d, seed=43).items()}
    oc, lc = binding.attention_forward(x["q"], x["k"], x["v"], True, scale)
    of, lf = binding.attention_forward(x["q"], x["k"], x["v"], False, scale)
    torch.cuda.synchronize()
    assert torch.equal(oc[:, 0], x["v"][:, 0])
    l0 = scale * (x["q"][:, 0].double() * x["k"][:, 0].double()).sum(-1)   # [B, H]
    assert (lc[:, :, 0].double() - l0).abs().max().item() < 1e-4
    _close(oc[:, -1], of[:, -1], "last row O")
    assert (lc[:, :, -1] - lf[:, :, -1]).abs().max().item() < 1e-3


@pytest.mark.parametrize("shape", SHAPES[:2], ids=IDS[:2])
def test_causal_prefix_consistency(shape):
    # causal rows i < M at length N see exactly the keys they see at length M
    B, H, N, d = shape
    M = N // 2 - 37
    scale = d ** -0.5
    x = {n: t.cuda() for n, t in make_inputs(B, H, N, d, seed=47).items()}
    o_n, l_n = binding.attention_forward(x["q"], x["k"], x["v"], True, scale)
    xm = {n: t[:, :M].contiguous() for n, t in x.items()}
    o_m, l_m = binding.attention_forward(xm["q"], xm["k"], xm["v"], True, scale)
    torch.cuda.synchronize()
    _close(o_n[:, :M], o_m, "prefix O")
    assert (l_n[:, :, :M] - l_m).abs().max().item() < 1e-3


@pytest.mark.parametrize("shape", SHAPES[:2], ids=IDS[:2])
def test_joint_key_value_permutation_leaves_full_attention_unchanged(shape):
    B, H, N, d = shape
    scale = d ** -0.5
    x = {n: t.cuda() for n, t in make_inputs(B, H, N, d, seed=53).items()}
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(5)).cuda()
    o1, l1 = binding.attention_forward(x["q"], x["k"], x["v"], False, scale)
    o2, l2 = binding.attention_forward(x["q"], x["k"][:, perm].contiguous(),
                                       x["v"][:, perm].contiguous(), False, scale)
    torch.cuda.synchronize()
    _close(o2, o1, "permuted O")
    assert (l1 - l2).abs().max().item() < 1e-3
