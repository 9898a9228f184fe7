"""Benchmark of the Q4_0 hot path on one MI355X.

Headline (the JSON line's ``value``): the decode GEMV, y[1, 4096] = a[1, 4096] @
dequant(W[4096, 4096])^T, as whole-job GB/s of algorithmic traffic (weight
blocks + activations + output) over K timed launches with the weights read
cold: each launch uses the next of R device copies of the weight blob, with R
copies spanning more than twice the 256 MiB last-level cache. One step is one
such GEMV. Inputs are resident in HBM before the timed region starts.

Every other row of the path is measured too and reported under ``rows``: the
8-row GEMV, the prefill GEMMs (1024 x 4096 x 4096 and 2048 x 14336 x 4096), the
dequant of the 14336 x 4096 weight and the Q8_0 quantize of a 2048 x 4096
tensor. Kernel durations come from HIP events recorded on the launch stream
around each launch; the roofline fraction uses the kernel's algorithmic bytes
or flops over that duration.

The oracle (CPU, f64) is timed on this host's cores on a bounded sample of the
decode GEMV and reported as ``cpu_baseline``; it is a reference point only.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|headline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6      # MI355X dense f16 MFMA (no sparsity)
LLC_BYTES = 256 * 2 ** 20          # MI355X last-level (MALL) cache


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--rows", choices=["all", "headline"], default="all")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- helpers

class Timer:
    """Per-launch HIP event pairs on the current stream."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]

    def durations_ms(self):
        return np.array([s.elapsed_time(e) for s, e in self.ev])


def run_timed(torch, fn, steps, warmup, min_warm_s=0.3):
    """Warm up (>= warmup launches and >= min_warm_s), then time `steps`
    launches twice: once back to back (whole-job time), once with an event pair
    around each launch (kernel durations)."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    start.record()
    for k in range(steps):
        fn(k)
    end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    region_ms = start.elapsed_time(end)
    timer = Timer(torch, steps)
    for k in range(steps):
        timer.ev[k][0].record()
        fn(k)
        timer.ev[k][1].record()
    torch.cuda.synchronize()
    d = timer.durations_ms()
    return {"region_ms": region_ms, "wall_s": wall_s, "kernel_ms_mean": float(d.mean()),
            "kernel_ms_median": float(np.median(d)), "kernel_ms_min": float(d.min()),
            "kernel_ms_p90": float(np.percentile(d, 90))}


def copies_for_cold(nbytes):
    return max(2, int(np.ceil(2.2 * LLC_BYTES / max(nbytes, 1))))


# ------------------------------------------------------------------- rows

def make_q4_weight(torch, q4, wl, N, K, seed):
    w32 = torch.from_numpy(wl.weights_f32(seed, N, K)).cuda()
    blob = torch.empty(N * (K // 32) * 18, dtype=torch.uint8, device="cuda")
    q4.q4_quantize(w32, blob)
    torch.cuda.synchronize()
    del w32
    return blob


def bench_product(torch, q4, wl, name, steps, warmup, cold=True):
    s = wl.WORKLOADS[name]
    M, N, K = s["M"], s["N"], s["K"]
    blob = make_q4_weight(torch, q4, wl, N, K, s["w_seed"])
    a = torch.from_numpy(wl.activations_f32(s["a_seed"], M, K)).cuda()
    y = torch.empty(M * N, dtype=torch.float32, device="cuda")
    wbytes = blob.numel()
    R = copies_for_cold(wbytes) if cold else 1
    blobs = [blob] + [blob.clone() for _ in range(R - 1)]
    fn_entry = q4.q4_gemv if s["kind"] == "gemv" else q4.q4_gemm
    fn = lambda i: fn_entry(a, blobs[i % R], y, M, N, K)
    t = run_timed(torch, fn, steps, warmup)
    algo_bytes = wbytes + M * K * 4 + M * N * 4
    flops = 2.0 * M * N * K
    row = {"workload": name, "M": M, "N": N, "K": K, "kernel": "k_%s_q4_0" % s["kind"],
           "weight_copies": R, "cache": "cold" if R > 1 else "warm",
           "algorithmic_bytes": algo_bytes, "flops": flops, **t}
    kern_s = t["kernel_ms_mean"] * 1e-3
    row["kernel_GBs"] = algo_bytes / kern_s / 1e9
    row["kernel_TFLOPs"] = flops / kern_s / 1e12
    row["job_GBs"] = algo_bytes * steps / (t["region_ms"] * 1e-3) / 1e9
    row["job_TFLOPs"] = flops * steps / (t["region_ms"] * 1e-3) / 1e12
    if s["kind"] == "gemv":
        row["roofline"] = {"bound": "hbm", "achieved": row["kernel_GBs"], "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": row["kernel_GBs"] / HBM_PEAK_GBS}
    else:
        row["roofline"] = {"bound": "mfma", "achieved": row["kernel_TFLOPs"],
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": row["kernel_TFLOPs"] / MFMA_F16_PEAK_TFLOPS,
                           "note": "f16 MFMA dense peak; the two-term activation split "
                                   "issues 2 MFMA flops per useful flop"}
    del blobs, blob, a, y
    torch.cuda.empty_cache()
    return row


def bench_dequant(torch, q4, wl, steps, warmup):
    s = wl.WORKLOADS["dequant_14336x4096"]
    N, K = s["N"], s["K"]
    blob = make_q4_weight(torch, q4, wl, N, K, s["w_seed"])
    outs = [torch.empty(N * K, dtype=torch.float32, device="cuda") for _ in range(2)]
    fn = lambda i: q4.q4_dequant(blob, outs[i % 2])
    t = run_timed(torch, fn, steps, warmup)
    algo = blob.numel() + N * K * 4
    kern_s = t["kernel_ms_mean"] * 1e-3
    row = {"workload": "dequant_14336x4096", "kernel": "k_dequant_q4_0", "cache": "cold",
           "algorithmic_bytes": algo, **t, "kernel_GBs": algo / kern_s / 1e9,
           "job_GBs": algo * steps / (t["region_ms"] * 1e-3) / 1e9}
    row["roofline"] = {"bound": "hbm", "achieved": row["kernel_GBs"], "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": row["kernel_GBs"] / HBM_PEAK_GBS}
    del blob, outs
    torch.cuda.empty_cache()
    return row


def bench_quantize(torch, q4, wl, steps, warmup):
    s = wl.WORKLOADS["quantize_2048x4096"]
    n = s["M"] * s["K"]
    x = torch.from_numpy(wl.activations_f32(s["x_seed"], s["M"], s["K"])).cuda().reshape(-1)
    R = copies_for_cold(n * 4)
    xs = [x] + [x.clone() for _ in range(R - 1)]
    out = torch.empty(n // 32 * 34, dtype=torch.uint8, device="cuda")
    fn = lambda i: q4.q8_quantize(xs[i % R], out)
    t = run_timed(torch, fn, steps, warmup)
    algo = n * 4 + n // 32 * 34
    kern_s = t["kernel_ms_mean"] * 1e-3
    row = {"workload": "quantize_2048x4096", "kernel": "k_quantize_q8_0", "input_copies": R,
           "cache": "cold", "algorithmic_bytes": algo, **t, "kernel_GBs": algo / kern_s / 1e9,
           "job_GBs": algo * steps / (t["region_ms"] * 1e-3) / 1e9}
    row["roofline"] = {"bound": "hbm", "achieved": row["kernel_GBs"], "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": row["kernel_GBs"] / HBM_PEAK_GBS}
    del xs, x, out
    torch.cuda.empty_cache()
    return row


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(wl, seconds):
    """The oracle (plain C, f64 sums, OpenMP over outputs) on this host, timed
    on repeated full decode GEMVs (1 x 4096 x 4096) for about `seconds`."""
    import oracle
    s = wl.WORKLOADS["gemv_1x4096x4096"]
    M, N, K = s["M"], s["N"], s["K"]
    blob = oracle.q4_0_quantize(wl.weights_f32(s["w_seed"], N, K))
    a = wl.activations_f32(s["a_seed"], M, K)
    threads = oracle.max_threads()
    oracle.q4_0_matmul(a, blob, N, K, threads=threads)          # warm
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        oracle.q4_0_matmul(a, blob, N, K, threads=threads)
        reps += 1
    el = time.perf_counter() - t0
    algo = blob.size + M * K * 4 + M * N * 4
    return {"value": algo * reps / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full 1x4096x4096 decode GEMVs in %.1f s (%.2f ms each), f64 sums"
                      % (reps, el, 1e3 * el / reps)}


# -------------------------------------------------------------------- main

def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding design); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_weight_dequant_amd import binding as q4
    from block_quantized_weight_dequant_amd import workloads as wl

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log("device: %s (%s), %d CUs" % (props.name, getattr(props, "gcnArchName", "?"),
                                      props.multi_processor_count))

    log("headline: decode GEMV 1x4096x4096, cold weights")
    head = bench_product(torch, q4, wl, "gemv_1x4096x4096", args.steps, args.warmup)
    rows = []
    if args.rows == "all":
        for name, st in (("gemv_8x4096x4096", args.steps), ("gemm_1024x4096x4096", 50),
                         ("gemm_2048x14336x4096", 20)):
            log("row: %s" % name)
            rows.append(bench_product(torch, q4, wl, name, min(st, args.steps),
                                      min(args.warmup, 10)))
        log("row: warm-cache decode GEMV")
        warm = bench_product(torch, q4, wl, "gemv_1x4096x4096", args.steps, args.warmup,
                             cold=False)
        warm["workload"] = "gemv_1x4096x4096_warm"
        rows.append(warm)
        log("row: dequant 14336x4096")
        rows.append(bench_dequant(torch, q4, wl, min(50, args.steps), min(args.warmup, 10)))
        log("row: Q8_0 quantize 2048x4096")
        rows.append(bench_quantize(torch, q4, wl, args.steps, args.warmup))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cpu = cpu_baseline(wl, args.cpu_seconds)

    value = head["job_GBs"]
    line = {
        "metric": "Q4_0 GEMV GB/s (M=1, 4096²) + prefill GEMM TFLOP/s, % of roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["region_ms"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 in/out; f16x2-split MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "gemv_1x4096x4096", "M": 1, "N": 4096, "K": 4096,
                   "cache": head["cache"], "weight_copies": head["weight_copies"]},
        "roofline": {**head["roofline"], "traffic": None,
                     "kernel": head["kernel"], "kernel_us_mean": head["kernel_ms_mean"] * 1e3,
                     "kernel_us_median": head["kernel_ms_median"] * 1e3},
        "cpu_baseline": cpu,
        "rows": rows,
        "device": props.name,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
