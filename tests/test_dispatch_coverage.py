"""Every kernel configuration the host dispatch can pick is compared with the
oracle by at least one GPU parity case.

fa2_fwd and fa2_bwd choose among kernel templates (waves per workgroup,
paired or dealt causal work) by problem size; a configuration no parity case
reaches would run untested.  fa2_fwd_variant / fa2_bwd_variant give the
dispatch's choice from the sizes alone (host arithmetic, no GPU), so this
runs on the CPU over the case lists the GPU parity modules run.  The d = 128
causal choice also depends on how many workgroups of one kernel a CU holds
at once; 2 is what gfx950 gives it (64 KB of LDS and at most 256 VGPRs per
4-wave workgroup), and test_parity_fwd repeats the check on the GPU with the
device's own answer.
"""
from exact_tiled_attention_30_amd import binding
from test_parity_bwd import bwd_parity_cases
from test_parity_fwd import fwd_parity_cases

GFX950_RESIDENT = 2


def test_every_forward_configuration_has_a_parity_case():
    seen = {binding.fa2_fwd_variant(*c, resident_wgs=GFX950_RESIDENT)
            for c in fwd_parity_cases()}
    missing = [binding.fa2_variant_name(v) for v in range(12) if v not in seen]
    assert not missing, missing


def test_every_backward_configuration_has_a_parity_case():
    seen = {binding.fa2_bwd_variant(*c) for c in bwd_parity_cases()}
    missing = [binding.fa2_variant_name(v) for v in range(16, 24) if v not in seen]
    assert not missing, missing


def test_variant_ids_and_names():
    names = [binding.fa2_variant_name(v) for v in list(range(12)) + list(range(16, 24))]
    assert all(names) and len(set(names)) == len(names)
    assert binding.fa2_variant_name(12) == "" and binding.fa2_variant_name(-1) == ""
    # invalid or empty problems have no configuration
    assert binding.fa2_fwd_variant(1, 1, 128, 96, False) == -1
    assert binding.fa2_fwd_variant(1, 0, 128, 64, True) == -1
    assert binding.fa2_bwd_variant(-1, 1, 128, 64, True) == -1
    # the documented picks of the measured workloads
    assert binding.fa2_variant_name(binding.fa2_fwd_variant(1, 16, 32768, 128, True, 2)) == \
        "fwd_dl_kernel<128,128,8,2,true>"
    assert binding.fa2_variant_name(binding.fa2_fwd_variant(4, 16, 4096, 128, False)) == \
        "fwd_sp_kernel<128,64,8>"
    assert binding.fa2_variant_name(binding.fa2_bwd_variant(4, 16, 4096, 128, True)) == \
        "bwd_dq_kernel<128,8,true>+bwd_kv_pair_kernel<128,true>"
