#!/usr/bin/env python3
"""Throughput of the FlashAttention-2 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step is one pass of the hot path over one batch of resident, seeded
synthetic inputs.  The default workload is the largest single-GPU one: the
long-context causal forward B=1, H=16, N=32768, d=128 with 1 % of the key rows
scaled by 8 (peaked softmax rows); a step is one fa2_fwd call.  Other
workloads (exact_tiled_attention_30_amd.inputs.WORKLOADS) can be named with
--workload, or the pair "fwd_b8_h16_n1024_d64_full+fwd_b8_h16_n1024_d64_causal"
(both masks on the same inputs); a backward workload's step is one fa2_bwd
call on O and L produced by fa2_fwd beforehand.

Before the W warm-up steps the step runs back to back for at least
--clock-warmup-ms of GPU time (reported as "clock_warmup_ms"): the GPU's clock
takes tens of milliseconds to settle, and a kernel timed before that reads
15-20 % slow.

FLOPs follow the usual convention: 4*B*H*N^2*d per forward, halved if causal;
a backward pass counts 2.5x its forward.  Timing uses HIP events on the stream
the kernels are launched on.  Inside the timed region the K steps are issued
grouped by launch (K calls of one kernel back to back, then the next), with an
event pair around each group, so each kernel's average duration is measured
there as well.

Prints ONE JSON line.  Besides the throughput it carries:
  roofline      the dominant kernel's achieved TFLOP/s against the bf16 dense
                MFMA peak, and against the MFMA throughput a plain MFMA loop
                reaches at the running clock (measured in the same run), and
                its HBM traffic from the committed rocprofv3 counter summary
                (null when the kernel source changed since);
  cpu_baseline  the fp64 oracle timed on the host cores on a bounded sample of
                the same workload (rows of a forward, whole heads of a
                backward), scaled to TFLOP/s;
  parity        the timed kernel's own outputs on that sample against the
                oracle's (oracle/compare.py), with the bare max |dO| <= 1e-2
                verdict beside the ulp-aware one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (4BHN²d, ½ if causal) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 bf16 FLOP/clk/CU x 2.4 GHz (dense)
DEFAULT_WORKLOAD = "fwd_b1_h16_n32768_d128_causal_peaked"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


KERNEL_SOURCES = {
    False: ("fa2_device.hpp", "fa2_internal.hpp", "fa2_fwd_kernels.hpp", "fa2_fwd.hip",
            "fa2_fwd_wide.hip"),
    True: ("fa2_device.hpp", "fa2_internal.hpp", "fa2_bwd.hip"),
}


def kernel_source_digest(backward: bool) -> str:
    """Digest of the sources of the forward (or backward) kernels; counter
    figures taken on one build are tied to it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_30_amd", "csrc")
    for name in KERNEL_SOURCES[backward]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, backward: bool):
    """HBM bytes per launch measured by rocprofv3 for this kernel, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(kernel_key)
    if not entry or entry.get("source_digest") != kernel_source_digest(backward):
        return None
    return entry.get("bytes_per_launch")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--clock-warmup-ms", type=float, default=300.0,
                   help="GPU time the step runs back to back before the warm-up steps, "
                        "so the clock has settled when timing starts")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD,
                   help="a workload name, or two forward workloads on the same inputs "
                        "joined by '+'")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    p.add_argument("--algo", choices=("fa2", "split-kv", "fa1-order", "fa1-split-k"),
                   default="fa2",
                   help="forward workloads: fa2_fwd, fa2_fwd_split_kv (library's slice "
                        "count), or the FlashAttention-1-order ablation fa2_fwd_fa1_order "
                        "with split-Q waves (fa1-order) or FlashAttention-1's split-K waves "
                        "(fa1-split-k)")
    p.add_argument("--bwd-dq", choices=("two-pass", "atomic"), default="two-pass",
                   help="dQ strategy of a backward workload: fa2_bwd (a Q-outer dQ pass) "
                        "or fa2_bwd_atomic_dq (fp32 atomics)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--memory", action="store_true",
                   help="only report the device memory of one forward + backward at "
                        "N = 4K, 16K, 64K (B=1, H=16, d=128, causal) and exit")
    p.add_argument("--cold", action="store_true",
                   help="forward workloads: alternate between two resident input sets "
                        "(and two outputs), so consecutive calls do not find their "
                        "inputs in the 256 MiB last-level cache when a set is larger")
    p.add_argument("--zero-inputs", action="store_true",
                   help="diagnostic: every input tensor zero (no oracle baseline, no parity). "
                        "The kernels execute the same instructions on any data, but the GPU's "
                        "clock under its power cap depends on how many operand bits toggle; "
                        "compared with the default run this shows that dependence")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (for scaling the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain device-to-device copy of known size, timed; under rocprofv3
    --pmc its FETCH_SIZE and WRITE_SIZE give the counters' scale factor."""
    import torch

    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    reps = 5
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps,
                      "ms": round(ms, 4), "GB_per_s": round(2 * n / ms / 1e6, 1)}), flush=True)


def measured_mfma_peak(stream, random_operands: bool = False, blocks: int = 2048,
                       iters: int = 4000) -> float:
    """bf16 MFMA TFLOP/s of the library's calibration kernel (two waves per
    SIMD issuing back-to-back MFMAs from registers), best of three timed
    calls after one warm-up: the attainable peak at the running clock.  With
    random_operands the operands change from one MFMA to the next as in an
    attention tile, which draws more power and so runs at a lower clock."""
    import torch

    from exact_tiled_attention_30_amd import binding

    fn = binding.fa2_calibrate_mfma_random if random_operands else binding.fa2_calibrate_mfma
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    fn(out, blocks, iters, stream.cuda_stream)
    flops = blocks * 4 * iters * 4 * 32768.0
    best = float("inf")
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(out, blocks, iters, stream.cuda_stream)
        b.record(stream)
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    return flops / (best * 1e-3) / 1e12


def activation_memory() -> None:
    """Device memory of one forward + backward through the library, against
    what a kernel that materialises the N x N matrices would hold.

    The library allocates nothing: every byte is a caller tensor, so the
    memory a training step keeps for the backward is O (bf16) and L (fp32),
    O(N) per head, where standard attention keeps P, O(N^2) per head.  The
    caller's tensors are allocated with torch and counted exactly; the device's
    free memory is read around the library calls to show they allocate
    nothing themselves."""
    import torch

    from exact_tiled_attention_30_amd import binding

    B, H, d = 1, 16, 128
    # one small call first: HIP loads the library's code object lazily
    x = torch.zeros((1, 64, 1, d), dtype=torch.bfloat16, device="cuda")
    ox, lx = binding.attention_forward(x, x, x, True)
    binding.attention_backward(x, x, x, ox, lx, x, True)
    torch.cuda.synchronize()
    for N in (4096, 16384, 65536):
        g = torch.Generator(device="cpu").manual_seed(0)
        q, k, v, do = (torch.randn((B, N, H, d), generator=g).to(torch.bfloat16).cuda()
                       for _ in range(4))
        o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(binding.fa2_bwd_workspace_bytes(B, H, N, d, True), dtype=torch.uint8,
                         device="cuda")
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        binding.fa2_fwd(q, k, v, o, lse, True, d ** -0.5)
        binding.fa2_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, True, d ** -0.5)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        nbytes = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
        saved = nbytes(o, lse)                     # kept from forward to backward
        total = nbytes(q, k, v, do, o, lse, dq, dk, dv, ws)
        std_p = B * H * N * N * 2                  # bf16 P kept for the backward
        print(json.dumps({
            "metric": "attention activation memory (fwd+bwd)", "N": N, "B": B, "H": H, "d": d,
            "causal": True, "saved_for_backward_bytes": saved,
            "all_tensors_bytes": total, "workspace_bytes": nbytes(ws),
            "library_allocated_bytes": int(free0 - free1),
            "standard_attention_P_bytes": std_p,
            "ratio_standard_over_saved": round(std_p / saved, 1)}), flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()


def main():
    args = parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.memory:
        activation_memory()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads shard with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from exact_tiled_attention_30_amd import binding
    from exact_tiled_attention_30_amd.inputs import inputs_for, workload

    names = tuple(args.workload.split("+"))
    ws = [workload(n) for n in names]
    base = ws[0]
    for w in ws[1:]:
        assert (w.B, w.H, w.N, w.d) == (base.B, base.H, base.N, base.d)

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    host = inputs_for(base)
    if args.zero_inputs:
        host = {n: torch.zeros_like(t) for n, t in host.items()}
        args.no_cpu = True
    x = {n: t.to(dev) for n, t in host.items()}
    o = torch.empty_like(x["q"])
    lse = torch.empty((base.B, base.H, base.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    launches = []  # (label, callable, flops)
    for w in ws:
        if not w.backward and args.algo == "split-kv":
            sws = torch.empty(binding.fa2_fwd_split_kv_workspace_bytes(w.B, w.H, w.N, w.d,
                                                                       w.causal, 0),
                              dtype=torch.uint8, device=dev)

            def fwd(w=w, sws=sws):
                binding.fa2_fwd_split_kv(x["q"], x["k"], x["v"], o, lse, sws, w.causal, w.scale, 0)
            launches.append((w.name, fwd, w.flops()))
        elif not w.backward and args.algo in ("fa1-order", "fa1-split-k"):
            fws = torch.empty(binding.fa2_fwd_fa1_order_workspace_bytes(w.B, w.H, w.N, w.d,
                                                                        w.causal),
                              dtype=torch.uint8, device=dev)

            def fwd(w=w, fws=fws):
                binding.fa2_fwd_fa1_order(x["q"], x["k"], x["v"], o, lse, fws, w.causal, w.scale,
                                          args.algo == "fa1-split-k")
            launches.append((w.name, fwd, w.flops()))
        elif not w.backward and args.cold:
            # a second input set (the same recipe, every value negated: the
            # same statistics, different bytes) and a second output
            x2 = {n: -t for n, t in x.items()}
            o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
            sets = [(x, o, lse), (x2, o2, lse2)]
            turn = [0]

            def fwd(w=w, sets=sets, turn=turn):
                xi, oi, li = sets[turn[0]]
                turn[0] ^= 1
                binding.fa2_fwd(xi["q"], xi["k"], xi["v"], oi, li, w.causal, w.scale)
            launches.append((w.name, fwd, w.flops()))
        elif not w.backward:
            def fwd(w=w):
                binding.fa2_fwd(x["q"], x["k"], x["v"], o, lse, w.causal, w.scale)
            launches.append((w.name, fwd, w.flops()))
        else:
            binding.fa2_fwd(x["q"], x["k"], x["v"], o, lse, w.causal, w.scale)
            dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
            atomic = args.bwd_dq == "atomic"
            sizer = (binding.fa2_bwd_atomic_dq_workspace_bytes if atomic
                     else binding.fa2_bwd_workspace_bytes)
            call = binding.fa2_bwd_atomic_dq if atomic else binding.fa2_bwd
            wsp = torch.empty(sizer(w.B, w.H, w.N, w.d, w.causal), dtype=torch.uint8,
                              device=dev)

            def bwd(w=w, dq=dq, dk=dk, dv=dv, wsp=wsp, call=call):
                call(x["q"], x["k"], x["v"], o, lse, x["dout"], dq, dk, dv, wsp, w.causal,
                     w.scale)
            launches.append((w.name, bwd, w.flops()))

    # clock warm-up: whole steps back to back until enough GPU time has passed
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    clock_warm_steps = 0
    while (time.perf_counter() - w0) * 1e3 < args.clock_warmup_ms:
        for _ in range(4):
            for _, fn, _ in launches:
                fn()
        clock_warm_steps += 4
        torch.cuda.synchronize()
    clock_warm_ms = (time.perf_counter() - w0) * 1e3
    for _ in range(args.warmup):
        for _, fn, _ in launches:
            fn()
    torch.cuda.synchronize()

    # The K steps are issued grouped by launch: K back-to-back calls of the
    # first launch, then K of the next.  An event pair brackets each group, so
    # a kernel's average duration carries no event packets between its calls.
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in launches]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for j, (_, fn, _) in enumerate(launches):
        ev[j][0].record(stream)
        for _ in range(K):
            fn()
        ev[j][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()

    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    step_flops = sum(f for _, _, f in launches)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    per_kernel_ms = [a.elapsed_time(b) / K for a, b in ev]
    dom = int(np.argmax(per_kernel_ms))
    dom_name, _, dom_flops = launches[dom]
    achieved = dom_flops / (per_kernel_ms[dom] * 1e-3) / 1e12

    peak_clock = measured_mfma_peak(stream)
    peak_random = measured_mfma_peak(stream, random_operands=True)

    roofline = {
        "bound": "mfma",
        "kernel": dom_name,
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": load_traffic(dom_name, ws[dom].backward),
        "avg_launch_ms": round(per_kernel_ms[dom], 5),
        "flops_per_launch": dom_flops,
        # the same kernel against what plain back-to-back MFMAs reach at the
        # clock the GPU runs at (fa2_calibrate_mfma, timed right after) ...
        "peak_measured": round(peak_clock, 1),
        "frac_of_measured": round(achieved / peak_clock, 4),
        # ... and when their operands change like an attention tile's
        # (fa2_calibrate_mfma_random): the power cap then lowers the clock
        "peak_measured_random": round(peak_random, 1),
        "frac_of_measured_random": round(achieved / peak_random, 4),
    }

    if args.no_cpu:
        cpu = parity = None
    elif ws[0].backward:
        cpu, parity = cpu_baseline_backward(ws[0], host, (dq, dk, dv))
    else:
        cpu, parity = cpu_baseline(ws, host, args.cpu_seconds, o, lse)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "clock_warmup_ms": round(clock_warm_ms, 1),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "zeros (clock diagnostic)" if args.zero_inputs else "synthetic",
        "config": {
            "workload": "+".join(w.name for w in ws),
            "B": base.B, "H": base.H, "N": base.N, "d": base.d,
            "causal": [w.causal for w in ws],
            "backward": [w.backward for w in ws],
            **({"bwd_dq": args.bwd_dq} if any(w.backward for w in ws) else {}),
            **({"algo": args.algo} if args.algo != "fa2" else {}),
            **({"inputs": "two resident sets, alternated (cold cache)"} if args.cold else {}),
            "layout": "[B,N,H,d] bf16 in/out, fp32 lse [B,H,N]",
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "per_kernel": {n: {"ms": round(t, 5),
                           "tflops": round(f / (t * 1e-3) / 1e12, 2)}
                       for (n, _, f), t in zip(launches, per_kernel_ms)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(ws, host, target_s, o_gpu, lse_gpu):
    """Time the fp64 oracle on a bounded sample of rows of the same workload,
    and compare the GPU's outputs on those rows with it.

    Rows are independent, so the FLOPs of a sample are exact: 4*n_vis*d per
    row (n_vis visible keys).  Inputs are widened to fp64 once, outside the
    timed calls; the sample size comes from a short calibration run.  o_gpu /
    lse_gpu hold the outputs of the step's last launch, which is compared.
    """
    import numpy as np
    import torch

    import oracle
    from oracle.compare import forward_report

    n_thr = oracle.num_threads()
    rng = np.random.default_rng(0)
    q64, k64, v64 = (oracle.widen(host[n]) for n in ("q", "k", "v"))

    def rows_for(w, n):
        return np.stack([rng.integers(w.B, size=n), rng.integers(w.H, size=n),
                         rng.integers(w.N, size=n)], 1)

    def flops(w, rows):
        nv = rows[:, 2] + 1 if w.causal else np.full(len(rows), w.N)
        return float(4.0 * nv.sum() * w.d)

    def timed(w, rows):
        t0 = time.perf_counter()
        ref = oracle.attention_forward_rows(q64, k64, v64, w.causal, w.scale, rows)
        return time.perf_counter() - t0, ref

    calib = max(32, 4 * n_thr)
    cal_f = cal_t = 0.0
    for w in ws:
        rows = rows_for(w, calib)
        cal_t += timed(w, rows)[0]
        cal_f += flops(w, rows)
    rate = cal_f / max(cal_t, 1e-9)

    total_f = total_t = 0.0
    desc = []
    parity = None
    for j, w in enumerate(ws):
        per_row = 4.0 * (w.N / 2 if w.causal else w.N) * w.d
        n = int(min(w.B * w.H * w.N, max(calib, target_s / len(ws) * rate / per_row)))
        rows = rows_for(w, n)
        t, (o_ref, lse_ref) = timed(w, rows)
        total_t += t
        total_f += flops(w, rows)
        desc.append(f"{n} random rows of {w.name}")
        if j == len(ws) - 1:
            b, h, i = (torch.as_tensor(rows[:, c], device=o_gpu.device) for c in range(3))
            rep = forward_report(o_gpu[b, i, h].cpu(), lse_gpu[b, h, i].cpu(), o_ref, lse_ref)
            parity = {"workload": w.name, "rows": n, **rep}
    return {
        "value": round(total_f / total_t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": n_thr,
        "kind": "oracle",
        "sample": "; ".join(desc) + f"; fp64, {total_t:.1f} s of oracle compute",
    }, parity


def cpu_baseline_backward(w, host, grads_gpu):
    """Time the fp64 oracle's backward on whole heads of the workload (one
    head per OpenMP thread, so every core works), and compare the GPU's
    gradients of those heads with it.  FLOPs by the same convention as the
    GPU: 2.5x the forward's 4*N^2*d per head, halved if causal."""
    import numpy as np

    import oracle
    from oracle.compare import gradient_report

    n_thr = oracle.num_threads()
    rng = np.random.default_rng(0)
    n_heads = min(w.B * w.H, n_thr)
    pick = rng.choice(w.B * w.H, size=n_heads, replace=False)
    heads = sorted((int(x) // w.H, int(x) % w.H) for x in pick)
    widened = [oracle.widen(host[n]) for n in ("q", "k", "v", "dout")]
    t0 = time.perf_counter()
    ref = oracle.attention_backward(*widened, w.causal, w.scale, heads)
    t = time.perf_counter() - t0
    per_head = 2.5 * 4.0 * w.N * w.N * w.d * (0.5 if w.causal else 1.0)
    parity = {"workload": w.name, "heads": len(heads)}
    for name, g in zip(("dq", "dk", "dv"), grads_gpu):
        got = np.stack([g[b, :, h, :].double().cpu().numpy() for (b, h) in heads])
        rep = gradient_report(got, ref[name])
        parity[name] = {k: rep[k] for k in ("max_rel", "mean_rel", "ok")}
    parity["ok"] = all(parity[n]["ok"] for n in ("dq", "dk", "dv"))
    return {
        "value": round(per_head * len(heads) / t / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": n_thr,
        "kind": "oracle",
        "sample": f"{len(heads)} whole heads (b, h) of {w.name}, forward recomputed and "
                  f"backward; fp64, {t:.1f} s of oracle compute",
    }, parity


if __name__ == "__main__":
    main()
