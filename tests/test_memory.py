"""The library allocates no device memory: the forward and backward use only
the caller's tensors (infra-guide page "6.2 FlashAttention V2 in depth",
section 8.3: FlashAttention keeps O(N) activation memory per head where
standard attention keeps the O(N^2) matrices).  Checked on the GPU by reading
the device's free memory around the calls."""
import pytest
import torch

from exact_tiled_attention_30_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("atomic_dq", [False, True], ids=["two_pass", "atomic_dq"])
def test_library_allocates_no_device_memory(atomic_dq):
    B, H, N, d = 1, 8, 8192, 128
    g = torch.Generator(device="cpu").manual_seed(1)
    q, k, v, do = (torch.randn((B, N, H, d), generator=g).to(torch.bfloat16).cuda()
                   for _ in range(4))
    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    sizer = (binding.fa2_bwd_atomic_dq_workspace_bytes if atomic_dq
             else binding.fa2_bwd_workspace_bytes)
    ws = torch.empty(sizer(B, H, N, d, True), dtype=torch.uint8, device="cuda")
    bwd = binding.fa2_bwd_atomic_dq if atomic_dq else binding.fa2_bwd
    # first calls outside the measurement (HIP loads the code object lazily)
    binding.fa2_fwd(q, k, v, o, lse, True, d ** -0.5)
    bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, d ** -0.5)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        binding.fa2_fwd(q, k, v, o, lse, True, d ** -0.5)
        bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, d ** -0.5)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
    # the two-pass workspace is O(N) per head (D only); the atomic one adds
    # an fp32 copy of dQ
    if not atomic_dq:
        assert ws.numel() == (B * H * N * 4 + 255) // 256 * 256
