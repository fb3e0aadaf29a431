"""bench.py's contract: the FLOP convention, the one-GPU rule, the traffic
figures' tie to the kernel sources, the CPU baseline record (CPU), and the
JSON line of a short run on the GPU."""
import json
import os
import subprocess
import sys

import pytest
import torch

import bench
from exact_tiled_attention_30_amd.inputs import WORKLOADS, Workload, inputs_for

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_convention():
    # 4*B*H*N^2*d forward, halved if causal; the backward counts 2.5x its forward
    assert WORKLOADS["fwd_b8_h16_n1024_d64_full"].flops() == 4 * 8 * 16 * 1024 ** 2 * 64
    assert WORKLOADS["fwd_b8_h16_n1024_d64_causal"].flops() == 2 * 8 * 16 * 1024 ** 2 * 64
    bwd = WORKLOADS["bwd_b4_h16_n4096_d128_causal"]
    assert bwd.flops() == 2.5 * 2 * 4 * 16 * 4096 ** 2 * 128
    assert abs(bwd.flops() - 6.87e11) / 6.87e11 < 1e-3


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    key = "fwd_b8_h16_n1024_d64_full"
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({key: {"source_digest": bench.kernel_source_digest(False),
                                   "bytes_per_launch": 123}}))
    assert bench.load_traffic(key, False) == 123
    # counters taken on other sources, or missing, give no figure
    f.write_text(json.dumps({key: {"source_digest": "0" * 16, "bytes_per_launch": 123}}))
    assert bench.load_traffic(key, False) is None
    assert bench.load_traffic("no_such_kernel", False) is None
    f.write_text("not json")
    assert bench.load_traffic(key, False) is None


def test_cpu_baseline_record():
    # the parity leg is plumbing here: the "GPU" outputs are the oracle's own,
    # rounded to bf16 as the library's are, so they must pass
    import oracle

    w = WORKLOADS["fwd_b1_h1_n128_d64_full"]
    wc = Workload("fwd_b1_h1_n128_d64_causal", 1, 1, 128, 64, True)
    x = inputs_for(w)
    o_ref, lse_ref = oracle.attention_forward(x["q"], x["k"], x["v"], True, wc.scale)
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).float()
    rec, parity = bench.cpu_baseline([w, wc], x, 0.05, o, lse)
    assert set(rec) == {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    # the whole workload is small: every row is in the sample
    assert rec["sample"].startswith("128 random rows of fwd_b1_h1_n128_d64_full")
    assert parity["workload"] == wc.name and parity["ok"] and parity["rows"] == 128
    assert "max_abs_dO_le_1e-2" in parity
    # and a wrong output is reported as such
    rec, parity = bench.cpu_baseline([wc], x, 0.05, o * 1.1, lse)
    assert not parity["ok"]


def test_cpu_baseline_backward_record():
    import oracle

    w = Workload("bwd_b1_h3_n200_d64_causal", 1, 3, 200, 64, True, backward=True)
    x = inputs_for(w)
    ref = oracle.attention_backward(x["q"], x["k"], x["v"], x["dout"], True, w.scale)
    grads = [torch.from_numpy(ref[n]).reshape(1, 3, 200, 64).permute(0, 2, 1, 3)
             .contiguous().to(torch.bfloat16) for n in ("dq", "dk", "dv")]
    rec, parity = bench.cpu_baseline_backward(w, x, grads)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["cores"] >= 1
    assert "whole heads" in rec["sample"]
    assert parity["ok"] and parity["heads"] == min(3, rec["cores"])
    rec, parity = bench.cpu_baseline_backward(w, x, [grads[0], grads[1] * 1.2, grads[2]])
    assert not parity["ok"] and not parity["dk"]["ok"]


@pytest.mark.gpu
def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5",
                        "--warmup", "2", "--cpu-seconds", "1"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "parity", "clock_warmup_ms"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    # the largest single-GPU workload is the default
    assert d["config"]["workload"] == "fwd_b1_h16_n32768_d128_causal_peaked"
    assert d["clock_warmup_ms"] >= 300
    assert d["parity"]["ok"] and d["parity"]["rows"] > 0
    assert d["value"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 2516.6 and rf["unit"] == "TFLOP/s"
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # both calibration modes ran; changing operands never beat the data sheet
    assert 0 < rf["peak_measured_random"] <= rf["peak"] and 0 < rf["peak_measured"] <= rf["peak"]
    assert abs(rf["frac_of_measured_random"] - rf["achieved"] / rf["peak_measured_random"]) < 1e-3
    # HBM bytes from the committed counter runs, or null once the kernels changed
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
