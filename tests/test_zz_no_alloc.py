"""fa2_bwd_noalloc against fa2_bwd (GPU).

The entry point for callers that cannot allocate runs the same kernels as
fa2_bwd with the D vector in the library's static scratch instead of a
caller workspace.  Two calls in a row, the second on a smaller problem (so
the scratch holds the first call's D when the second starts), each compared
with fa2_bwd on the same inputs: bitwise equal, and within the gradient
tolerance of the fp64 oracle.  The device's free memory does not move across
the calls.
"""
import pytest
import torch

import oracle
from exact_tiled_attention_30_amd import binding
from exact_tiled_attention_30_amd.inputs import make_inputs
from oracle.compare import gradient_report

pytestmark = pytest.mark.gpu

# (B, H, N, d, causal): the second call is smaller than the first
CALLS = [(2, 4, 700, 128, True), (1, 3, 300, 64, False)]


def test_noalloc_backward_matches_fa2_bwd_on_two_calls():
    prepared = []
    for (B, H, N, d, causal) in CALLS:
        x = make_inputs(B, H, N, d, seed=41 + N, with_dout=True)
        dx = {n: t.cuda() for n, t in x.items()}
        o, lse = binding.attention_forward(dx["q"], dx["k"], dx["v"], causal, d ** -0.5)
        ref = binding.attention_backward(dx["q"], dx["k"], dx["v"], o, lse, dx["dout"], causal,
                                         d ** -0.5)
        outs = tuple(torch.empty_like(dx["q"]) for _ in range(3))
        prepared.append((x, dx, o, lse, ref, outs))
    # every tensor exists before the measured calls: only the library could
    # allocate between the two readings of the free memory
    binding.fa2_bwd_noalloc(*(torch.empty((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
                              for _ in range(4)),
                            torch.zeros((1, 1, 1), device="cuda"),
                            *(torch.empty((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
                              for _ in range(4)), True, 0.125)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for (B, H, N, d, causal), (x, dx, o, lse, ref, outs) in zip(CALLS, prepared):
        print(f"[noalloc] B={B} H={H} N={N} d={d} causal={causal}", flush=True)
        binding.fa2_bwd_noalloc(dx["q"], dx["k"], dx["v"], o, lse, dx["dout"], *outs, causal,
                                d ** -0.5)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
    for (B, H, N, d, causal), (x, dx, o, lse, ref, outs) in zip(CALLS, prepared):
        outs_h = [g.cpu() for g in outs]
        for name, a, b in zip(("dq", "dk", "dv"), outs_h, ref):
            assert torch.equal(a, b.cpu()), (name, (B, H, N, d, causal))
        heads = [(b, h) for b in range(B) for h in range(H)]
        want = oracle.attention_backward(x["q"], x["k"], x["v"], x["dout"], causal, d ** -0.5,
                                         heads)
        for name, g in zip(("dq", "dk", "dv"), outs_h):
            got = torch.stack([g[b, :, h, :] for (b, h) in heads]).double().numpy()
            rep = gradient_report(got, want[name])
            assert rep["ok"], (name, rep)


def test_noalloc_rejects_a_problem_past_its_scratch():
    # B*H*N one row past the static scratch: refused before any launch
    q = torch.empty((1, binding.BWD_NOALLOC_MAX_ROWS + 1, 1, 64), dtype=torch.bfloat16,
                    device="cuda")
    lse = torch.empty((1, 1, q.shape[1]), device="cuda")
    with pytest.raises(binding.Fa2Error, match="FA2_ERR_SCRATCH"):
        binding.fa2_bwd_noalloc(q, q, q, q, lse, q, *(torch.empty_like(q) for _ in range(3)),
                                True, 0.125)
