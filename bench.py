"""Benchmark of the KDA chunked forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload i]

A step is one kda_fwd call (chunk table, prep, state/output stages) over one batch of
seeded synthetic input already resident in HBM.  Default workload: the largest one, a single
1,048,576-token sequence with H=8, K=V=128, fp32 initial and final state (index 3 of
workloads.config).  Prints one JSON line.

W warm-up steps (default 100: a fresh process needs some 20 ms of sustained load before the
forward kernel reaches its steady speed) are not timed.
value and ms_per_step: K steps run back to back with nothing between the launches.  Then
K more steps with HIP events recorded on the launch stream around every launch give each
kernel's duration (recording an event between two launches delays the second one by a few
microseconds, so these steps are timed separately and reported as ms_per_step_with_events).
roofline: the dominant kernel, fused_kernel (the forward kernel), against HBM; for the
decode workload (--workload 5, one token per sequence) the step is kda_fwd_recurrent and
the dominant kernel is recurrent_kernel.  With a
whole-chain plan fused_kernel runs once per step; with the cut plan (long sequences)
three times, pass A, the transition runs and pass B, with seg_scan_kernel before pass B.  achieved = the path's algorithmic bytes per
step / fused_kernel's time per step (the sum over its launches): q, k, v, g (4 x 256 B) +
beta (2 B) + out (256 B) per head-token, plus initial/final state.  traffic (when the
committed rocprofv3 summary matches the kernel source) is fused_kernel's calibrated
FETCH_SIZE + WRITE_SIZE per step, summed the same way.
flushed: K more steps, each after writing a 1 GiB scratch buffer (which evicts the 4 MiB L2
of every XCD and the 256 MiB MALL), each timed alone with HIP events: median, p10, p90.
Workloads whose bytes exceed the MALL many times over (the 2^20-token one moves 10.8 GB)
time the same either way; the small ones would otherwise run out of the MALL.
cpu_baseline: the fp64 oracle on the host cores, on a bounded sample of the same workload.

--copy-calibration runs only a plain device-to-device copy of known size (for scaling the
FETCH_SIZE / WRITE_SIZE hardware counters); it prints the bytes copied per launch.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
BYTES_PER_HT = 1282              # q, k, v, g (4 x 256) + beta (2) + out (256)
FLOPS_PER_HT = 122880            # dense contractions per head-token (three 16x128x128 per chunk + intra-chunk)
METRIC = "KDA fwd head-tokens/sec on 1 MI355X + % of HBM/MFMA roofline"
# backward: q, k, v, g (4 x 256) + beta (2) + dL/dout (256) in; dq, dk, dv, dg (4 x 512, fp32) +
# dbeta (4) out
BWD_BYTES_PER_HT = 3334
DECODE_WORKLOADS = (5,)          # run through the token-by-token entry point (kda_fwd_recurrent)


def state_bytes(w):
    per = 128 * 128
    b = 0
    if w.initial_state is not None:
        b += w.N * w.H * per * (2 if w.state_dtype == "bf16" else 4)
    if w.final_dtype != "none":
        b += w.N * w.H * per * (2 if w.final_dtype == "bf16" else 4)
    return b


def committed_traffic(workload_name, kernel, source="kda_kernels.hip", pass_="fwd"):
    """HBM bytes per step of `kernel` (summed over its launches; for the backward pass, "kda_bwd":
    every kernel of the pass) from the committed rocprofv3 summary of this workload
    (profiles/kda_<pass_>_<workload>.md), or None when there is none or the kernel source has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"kda_{pass_}_{workload_name}.md")
    src = os.path.join(ROOT, "gated_delta_rule_86_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for line in open(path):
        if line.startswith("traffic_bytes_per_step:"):
            fields = dict(f.split("=", 1) for f in line.split(":", 1)[1].split() if "=" in f)
            if fields.get("source_sha256") == sha and kernel in fields:
                try:
                    return int(fields[kernel])
                except ValueError:
                    return None
    return None


def committed_counter(workload_name, key, kernel, source="kda_kernels.hip"):
    """A per-kernel figure (a float) from the line `<key>: <kernel>=<x> ... source_sha256=...`
    of the committed profile of this workload, or None when there is none or the kernel source
    has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"kda_fwd_{workload_name}.md")
    src = os.path.join(ROOT, "gated_delta_rule_86_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for line in open(path):
        if line.startswith(key + ":"):
            fields = dict(f.split("=", 1) for f in line.split(":", 1)[1].split() if "=" in f)
            if fields.get("source_sha256") == sha and kernel in fields:
                try:
                    return float(fields[kernel])
                except ValueError:
                    return None
    return None


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def copy_calibration(steps):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n, "bytes_written_per_launch": n,
                                           "launches": steps}}), flush=True)


def cpu_baseline(w):
    import numpy as np

    import oracle
    from gated_delta_rule_86_amd import workloads as W
    oracle.build()
    threads = oracle.max_threads()
    chains = w.N * w.H
    if w.head_tokens <= 3_000_000:
        ws, sample = w, "the whole workload"
    else:  # first T' tokens of every sequence of a single long batch row
        Tp = max(16, 2_000_000 // (w.H * w.B))
        sl = lambda a: np.ascontiguousarray(a[:, :Tp])
        ws = W.Workload(w.name, w.B, Tp, w.H, sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), w.A_log,
                        w.dt_bias, w.lower_bound, w.scale, w.initial_state, w.state_dtype, w.final_dtype,
                        None)
        sample = f"first {Tp} tokens of each of the {w.B * w.H} (row, head) chains"
    t0 = time.perf_counter()
    oracle.kda_fwd(ws.q, ws.k, ws.v, ws.g, ws.beta, ws.scale, ws.A_log, ws.dt_bias, ws.lower_bound,
                   ws.initial_state, cu_seqlens=ws.cu_seqlens)
    dt = time.perf_counter() - t0
    return {"value": ws.head_tokens / dt, "unit": "head-tokens/s", "cores": min(threads, chains),
            "kind": "oracle", "sample": f"{sample} ({ws.head_tokens} head-tokens, {dt:.2f} s wall; one "
            f"thread per chain, {min(threads, chains)} of the {threads} available)"}


def backward_bench(args, w):
    """Time kda_bwd on the workload's inputs with a random dL/dout and dL/dfinal_state; one JSON
    line (head-tokens/s of the backward pass; not the headline metric)."""
    import numpy as np
    import torch
    from gated_delta_rule_86_amd import kda
    from gated_delta_rule_86_amd import workloads as W
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).to(dev)
    q, k, v, g, beta = (t(getattr(w, n)) for n in ("q", "k", "v", "g", "beta"))
    A_log = torch.from_numpy(w.A_log).to(dev)
    dt_bias = torch.from_numpy(w.dt_bias).to(dev)
    h0 = None
    if w.initial_state is not None:
        h0 = t(w.initial_state) if w.initial_state.dtype.name == "uint16" else torch.from_numpy(w.initial_state).to(dev)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev)
    rng = np.random.default_rng(0)
    dout = t(W.f32_to_bf16_bits(rng.standard_normal(q.shape, dtype=np.float32)))
    dht = torch.randn((w.N, w.H, 128, 128), device=dev)
    ws = torch.empty(kda.bwd_workspace_size(w.B, w.T, w.H, w.N, cu is not None), dtype=torch.uint8, device=dev)
    step = lambda: kda.bwd(q, k, v, g, beta, w.scale, A_log, dt_bias, w.lower_bound, dout, h0, dht, cu,
                           workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    # algorithmic bytes: the per-token tensors, plus per chain the initial state and
    # dL/dfinal_state in and dL/dinitial_state out (fp32)
    per = w.N * w.H * 128 * 128
    h0_bytes = 0 if w.initial_state is None else per * (2 if w.state_dtype == "bf16" else 4)
    path_bytes = w.head_tokens * BWD_BYTES_PER_HT + h0_bytes + 2 * 4 * per
    achieved = path_bytes / dt / 1e9
    print(json.dumps({"metric": "KDA bwd head-tokens/sec on 1 MI355X (kda_bwd)", "value": w.head_tokens / dt,
                      "unit": "head-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": dt * 1e3, "higher_is_better": True, "dtype": "fp32",
                      "data": "synthetic", "config": dict(w.describe(), head_tokens=w.head_tokens),
                      "roofline": {"bound": "hbm", "achieved": achieved, "peak": 8000.0, "unit": "GB/s",
                                   "frac": achieved / 8000.0,
                                   "traffic": committed_traffic(w.name, "kda_bwd", "kda_backward.hip", "bwd"),
                                   "kernel": "kda_bwd, all launches (chunk records, operands, the two walks (whole or cut plan with its scan), gradients, head sums)",
                                   "algorithmic_bytes": path_bytes},
                      "workspace_bytes": ws.numel()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU needs some 20 ms of sustained load before the forward kernel reaches its steady
    # speed (the first launches of a fresh process run 6-9 % slower); 100 steps cover that
    # for every workload here
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=3,
                    help="index into workloads.config (0..4; 5 = decode step, token-by-token path)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time kda_bwd (gradients of out and final_state) on the workload instead")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (got --gpus {args.gpus}); the (sequence, "
              "head) chains shard across GPUs with no communication, but no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    from gated_delta_rule_86_amd import kda
    from gated_delta_rule_86_amd import workloads as W

    w = W.config(args.workload)
    if args.backward:
        backward_bench(args, w)
        return
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    q, k, v, g, beta = (t(getattr(w, n)) for n in ("q", "k", "v", "g", "beta"))
    A_log = torch.from_numpy(w.A_log).to(dev)
    dt_bias = torch.from_numpy(w.dt_bias).to(dev)
    h0 = None
    if w.initial_state is not None:
        h0 = t(w.initial_state) if w.initial_state.dtype.name == "uint16" else torch.from_numpy(w.initial_state).to(dev)
    cu = None if w.cu_seqlens is None else torch.from_numpy(w.cu_seqlens).to(dev)
    out = torch.empty_like(q)
    fin = None
    if w.final_dtype != "none":
        fin = torch.empty((w.N, w.H, 128, 128), device=dev,
                          dtype=torch.float32 if w.final_dtype == "fp32" else torch.bfloat16)
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.N, cu is not None), dtype=torch.uint8, device=dev)

    recurrent = args.workload in DECODE_WORKLOADS
    entry = kda.fwd_recurrent if recurrent else kda.fwd

    def step(events=None):
        entry(q, k, v, g, beta, w.scale, out, A_log, dt_bias, w.lower_bound, h0, fin, cu,
              workspace=ws, stage_events=events)

    hip = hip_runtime()
    ev = []
    for _ in range(args.steps):
        row = []
        for _ in range(5):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            row.append(e.value)
        ev.append(row)

    for _ in range(args.warmup):
        step()
    # value: K steps exactly as a caller runs them (no events between the launches)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-launch durations: K more steps with HIP events recorded around every launch on the
    # launch stream (the event records sit between the launches, so these steps are not the
    # ones the throughput comes from)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1

    # intervals: table, pass A (+ transition runs) or the one forward launch, scan, pass B
    iv = [0.0, 0.0, 0.0, 0.0]
    for i in range(args.steps):
        for j in range(2 if recurrent else 4):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[i][j], ev[i][j + 1]) == 0
            iv[j] += ms.value / args.steps
    if recurrent:  # events: before the table, before the recurrent kernel, after it
        launches = 1
        stage_names = ["chunk_table_kernel", "recurrent_kernel"]
        stage_ms = [iv[0], iv[1]]
    else:
        launches = kda.forward_launches(w.B, w.T, w.H, w.N, cu is not None)
        stage_names = ["chunk_table_kernel", "fused_kernel", "seg_scan_kernel"]
        if launches > 1:
            stage_ms = [iv[0], iv[1] + iv[3], iv[2]]
        else:  # one forward launch; the later marks are recorded back to back
            stage_ms = [iv[0], iv[1], 0.0]
    for row in ev:
        for e in row:
            hip.hipEventDestroy(e)

    # flushed steps: 1 GiB written before each, each step timed alone on the launch stream
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    fl_ms = []
    for i in range(args.steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        fl_ms.append(e0.elapsed_time(e1))
    del flush
    fl_sorted = sorted(fl_ms)
    pct = lambda p: fl_sorted[min(len(fl_sorted) - 1, max(0, int(round(p * (len(fl_sorted) - 1)))))]

    ht = w.head_tokens
    ms_per_step = elapsed / args.steps * 1e3
    value = ht / (elapsed / args.steps)
    dname = "recurrent_kernel" if recurrent else "fused_kernel"
    dsrc = "kda_recurrent.hip" if recurrent else "kda_kernels.hip"
    kernel_bytes = ht * BYTES_PER_HT + state_bytes(w)
    achieved = kernel_bytes / (stage_ms[1] * 1e-3) / 1e9
    path_bytes = ht * BYTES_PER_HT + state_bytes(w)
    path_gbps = path_bytes / (ms_per_step * 1e-3) / 1e9
    path_tflops = ht * FLOPS_PER_HT / (ms_per_step * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(w.describe(), head_tokens=ht),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": committed_traffic(w.name, dname, dsrc),
                     "kernel": dname, "launches_per_step": launches,
                     "kernel_ms": stage_ms[1], "kernel_algorithmic_bytes": kernel_bytes,
                     "frac_whole_step": path_gbps / HBM_PEAK_GBPS,
                     "mfma_busy_frac": committed_counter(w.name, "mfma_busy", dname, dsrc)},
        "timing": {"ms_per_step_with_events": elapsed_ev / args.steps * 1e3,
                   "flushed_ms_p50": pct(0.5), "flushed_ms_p10": pct(0.1), "flushed_ms_p90": pct(0.9),
                   "flushed_value_p50": ht / (pct(0.5) * 1e-3), "flush_bytes": 1 << 30},
        "path": {"algorithmic_bytes": path_bytes, "achieved_GBps": path_gbps,
                 "hbm_frac": path_gbps / HBM_PEAK_GBPS, "achieved_TFLOPs": path_tflops,
                 "mfma_frac": path_tflops / MFMA_BF16_PEAK_TFLOPS,
                 "stage_ms": dict(zip(stage_names, stage_ms))},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
