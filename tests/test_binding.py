"""The Python binding turns tensors into pointers only after checking them:
wrong dtypes, non-contiguous views, host tensors and malformed shapes raise
before any library call (CPU; no tensor here ever reaches the C ABI)."""
import pytest
import torch

from exact_tiled_attention_30_amd import binding

B, N, H, D = 1, 8, 2, 64


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def strided(t):
    """A non-contiguous view of the same shape and dtype."""
    wide = torch.zeros(t.shape[:-1] + (2 * t.shape[-1],), dtype=t.dtype)
    return wide[..., ::2]


def fwd_args():
    q, k, v, o = (bf16(B, N, H, D) for _ in range(4))
    lse = torch.zeros((B, H, N), dtype=torch.float32)
    return q, k, v, o, lse


def test_forward_rejects_bad_tensors():
    q, k, v, o, lse = fwd_args()
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        binding.fa2_fwd(q.float(), k, v, o, lse, False, 0.125)
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        # the bf16 tensors fail first on the host check, so give lse alone a bad dtype
        binding._require(lse.double(), torch.float32, "lse")
    with pytest.raises(ValueError, match="contiguous"):
        binding.fa2_fwd(strided(q), k, v, o, lse, False, 0.125)
    with pytest.raises(ValueError, match="device tensor"):
        binding.fa2_fwd(q, k, v, o, lse, False, 0.125)
    with pytest.raises(ValueError, match=r"\[B, N, H, d\]"):
        binding.fa2_fwd(q[0], k, v, o, lse, False, 0.125)
    with pytest.raises(ValueError, match="device tensor"):
        binding.attention_forward(q, k, v, True)


def test_backward_rejects_bad_tensors():
    q, k, v, o, lse = fwd_args()
    do, dq, dk, dv = (bf16(B, N, H, D) for _ in range(4))
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    for f in (binding.fa2_bwd, binding.fa2_bwd_atomic_dq):
        # the tensors are checked in order and the first failing one raises
        with pytest.raises(TypeError):
            f(q.half(), k, v, o, lse, do, dq, dk, dv, ws, True, 0.125)
        with pytest.raises(ValueError, match="contiguous"):
            f(strided(q), k, v, o, lse, do, dq, dk, dv, ws, True, 0.125)
        with pytest.raises(ValueError, match="device tensor"):
            f(q, k, v, o, lse, do, dq, dk, dv, ws, True, 0.125)
    with pytest.raises(ValueError, match="device tensor"):
        binding.attention_backward(q, k, v, o, lse, do, True)
    # lse: the kernels read B*H*N floats in [B, H, N] order, so a short lse or
    # one in another layout ([B, N, H] here) is refused before any library call
    for bad_lse in (torch.zeros((B, H, N - 1)), torch.zeros((B, N, H)), torch.zeros(B * H * N)):
        for f in (binding.fa2_bwd, binding.fa2_bwd_atomic_dq):
            with pytest.raises(ValueError, match=r"lse must have shape"):
                f(q, k, v, o, bad_lse, do, dq, dk, dv, ws, True, 0.125)
        with pytest.raises(ValueError, match=r"lse must have shape"):
            binding.fa2_fwd(q, k, v, o, bad_lse, False, 0.125)
    with pytest.raises(ValueError, match=r"dout must have shape"):
        binding.fa2_bwd(q, k, v, o, lse, do[:, :-1], dq, dk, dv, ws, True, 0.125)


def test_calibration_rejects_bad_output():
    for fn in (binding.fa2_calibrate_mfma, binding.fa2_calibrate_mfma_random):
        with pytest.raises(TypeError):
            fn(torch.zeros(256, dtype=torch.float64), 1, 1)
        with pytest.raises(ValueError, match="too small"):
            fn(torch.zeros(255, dtype=torch.float32), 1, 1)


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    # no libfa2.so: loading it raises, there is no other implementation to fall back to
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libfa2.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="is not built"):
        binding.lib()
    # and host tensors are rejected by the checks, never computed on the CPU
    q, k, v, _, _ = fwd_args()
    with pytest.raises(ValueError, match="device tensor"):
        binding.attention_forward(q, k, v, causal=True)
