"""Benchmark of the Q4_0 (and Q8_0-weight) hot path on one MI355X.

Headline (the JSON line's ``value``): the decode GEMV y[1, 4096] =
a[1, 4096] @ dequant(W[4096, 4096])^T, as whole-job GB/s of algorithmic
traffic (weight blocks + activations + output) over K timed steps. One step is
one GEMV. The weights are read cold: step k uses the (k mod R)-th of R device
copies of the weight blob, and the R copies span more than twice the 256 MiB
last-level cache. All inputs are resident in HBM before timing starts.

Timing: the K launches of a timed region are captured once into a HIP graph
(plain kernel nodes, no memset nodes) and replayed, so host submission cannot
starve the GPU; the region is bracketed by HIP events recorded on the launch
stream and by torch.cuda.synchronize() on both sides. A kernel's duration is
the event-measured region divided by K (back-to-back launches, so it includes
the inter-kernel gap and is never shorter than the kernel itself).

Every other row of the path is measured the same way and reported under
``rows``: the 8-row GEMV, the prefill GEMMs (1024 x 4096 x 4096 and
2048 x 14336 x 4096), a warm-cache GEMV, the dequant of the 14336 x 4096 weight
and the Q8_0 quantize of a 2048 x 4096 tensor; then the GEMVs, GEMMs and
dequant again over Q8_0 weights.

``roofline.traffic`` comes from the committed counter summary
profiles/traffic.json (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy of
known size) and is null when the kernel source has changed since.

The oracle (CPU, f64) is timed on this host's cores on repeated full decode
GEMVs for a bounded time and reported as ``cpu_baseline``.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|headline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6      # MI355X dense f16 MFMA (no sparsity)
LLC_BYTES = 256 * 2 ** 20          # MI355X last-level (MALL) cache
KERNEL_SOURCES = {
    "gemv": "block_quantized_weight_dequant_amd/csrc/gemv.hip",
    "gemm": "block_quantized_weight_dequant_amd/csrc/gemm.hip",
    "dequant": "block_quantized_weight_dequant_amd/csrc/dequant.hip",
    "quantize": "block_quantized_weight_dequant_amd/csrc/quantize.hip",
}


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--rows", choices=["all", "headline"], default="all")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a 256 MiB device copy (counter calibration)")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha256(kind):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kind]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(workload, kernel, kind):
    """Measured HBM bytes per launch (reads + writes) of `kernel` on `workload`,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["workloads"].get(workload)
    except (OSError, ValueError, KeyError):
        return None
    if not rec or rec.get("kernel") != kernel or rec.get("source_sha256") != source_sha256(kind):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------- timing

def run_timed(torch, fn, steps, warmup, min_warm_s=0.3):
    """Capture `steps` launches (fn(k), k = 0..steps-1) into one HIP graph, warm
    up by replaying it (>= warmup launches and >= min_warm_s), then time one
    replay with events on the current stream and the host clock."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(min(steps, 3)):
            fn(k)                                    # eager warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(steps):
            fn(k)
    done, t0 = 0, time.perf_counter()
    while done < warmup or time.perf_counter() - t0 < min_warm_s:
        graph.replay()
        done += steps
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - w0
    region_ms = start.elapsed_time(end)
    del graph
    return {"region_ms": region_ms, "wall_s": wall_s, "kernel_us": region_ms * 1e3 / steps,
            "steps": steps, "launch": "hip-graph replay of the timed launches"}


def copies_for_cold(nbytes):
    return max(2, int(np.ceil(2.2 * LLC_BYTES / max(nbytes, 1))))


def hbm_roofline(algo_bytes, kernel_us, workload, kernel, kind):
    achieved = algo_bytes / (kernel_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(workload, kernel, kind),
            "kernel": kernel}


# ------------------------------------------------------------------- rows

BLOCK_BYTES = {"q4_0": 18, "q8_0": 34}
FMT_TYPE = {"q4_0": "FmtQ4_0", "q8_0": "FmtQ8_0"}


def make_weight(torch, q4, wl, N, K, seed, fmt="q4_0"):
    """The workload's f32 weights quantized on the device (q4_quantize or
    q8_quantize)."""
    w32 = torch.from_numpy(wl.weights_f32(seed, N, K)).cuda()
    blob = torch.empty(N * (K // 32) * BLOCK_BYTES[fmt], dtype=torch.uint8, device="cuda")
    (q4.q4_quantize if fmt == "q4_0" else q4.q8_quantize)(w32, blob)
    torch.cuda.synchronize()
    del w32
    return blob


def digest(x) -> str:
    """SHA-256 of a generated input's bytes (a device tensor or a numpy array), so
    that the inputs behind a figure can be compared across runs and machines."""
    if hasattr(x, "cpu"):
        x = x.cpu().numpy()
    return hashlib.sha256(x.tobytes()).hexdigest()


def gemv_kernel_name(M, K, fmt="q4_0", act="f32", splitk=False, N=0, prepared=False):
    """The kernel the library launches (mirrors launch_gemv_m, launch_gemv_q8a_m and
    gemv_split_plan)."""
    if act == "q8_0":
        if K % 256:
            return "k_gemv_q8a_any<%s, %d>" % (FMT_TYPE[fmt], M)
        ch16 = (K // 32) % 16 == 0 and ((N + 15) // 16 <= 256 or M == 1)
        return "k_gemv_q8a<%s, %d, 8, %d>" % (FMT_TYPE[fmt], M, 16 if ch16 else 8)
    bf = "true" if act == "bf16" else "false"
    if K % 256:
        return "k_gemv<%s, %d, %s>" % (FMT_TYPE[fmt], M, bf)
    nblk = K // 32
    if prepared:
        return "k_gemv_stream<%s, %d, 8, %d, false, 2>" % (FMT_TYPE[fmt], M,
                                                           16 if nblk % 16 == 0 else 8)
    ks = kl = nblk
    if splitk:   # the library's automatic split
        groups = (N + 15) // 16
        want = min(-(-256 // groups), nblk // 64, nblk // 8)
        ch0 = 16 if nblk % 16 == 0 else 8
        if -(-(nblk // ch0) // 8) < 3:
            want = 1
        if want > 1:
            ks = (-(-nblk // want) + 7) & ~7
            kl = nblk - (-(-nblk // ks) - 1) * ks
    ch = 16 if (ks % 16 == 0 and kl % 16 == 0) else 8
    ni = M if act == "bf16" else 2 * M
    splits = -(-nblk // ks)
    al = ((N + 15) // 16 * splits > 256 or ks > 8 * ch) and not (ch == 16 and ni > 8)
    return "k_gemv_stream<%s, %d, 8, %d, %s, %d>" % (FMT_TYPE[fmt], M, ch, bf, 1 if al else 0)


def gemm_kernel_name(K, fmt="q4_0", act="f32"):
    if K % 64:
        return "k_gemm_any<%s>" % FMT_TYPE[fmt]
    return "k_gemm_split<%s, %s>" % (FMT_TYPE[fmt], "true" if act == "bf16" else "false")


def bench_product(torch, q4, wl, name, steps, warmup, cold=True):
    s = wl.WORKLOADS[name]
    M, N, K = s["M"], s["N"], s["K"]
    fmt = s.get("fmt", "q4_0")
    f = fmt[:2]
    act = s.get("act", "f32")
    blob = make_weight(torch, q4, wl, N, K, s["w_seed"], fmt)
    if act == "bf16":
        a = torch.from_numpy(wl.activations_bf16(s["a_seed"], M, K).view("int16")).cuda()
    else:
        a = torch.from_numpy(wl.activations_f32(s["a_seed"], M, K)).cuda()
    y = torch.empty(M * N, dtype=torch.float32, device="cuda")
    wbytes = blob.numel()
    R = copies_for_cold(wbytes) if cold else 1
    blobs = [blob] + [blob.clone() for _ in range(R - 1)]
    prep_us = quant_us = None
    if act == "q8_0":
        # The activations are quantized once, outside the timed region (its own
        # time is quant_us); the product reads the Q8_0 blocks.
        a_q = torch.empty(M * (K // 32) * 34, dtype=torch.uint8, device="cuda")
        q4.q8_quantize(a, a_q)
        if s["kind"] == "gemv":
            gemv = getattr(q4, f + "_gemv_q8a")
            fn = lambda k: gemv(a_q, blobs[k % R], y, M, N, K)
        else:
            gemm = getattr(q4, f + "_gemm_q8a")
            ws = torch.empty(max(getattr(q4, f + "_gemm_q8a_workspace_bytes")(M, N, K), 16),
                             dtype=torch.uint8, device="cuda")
            fn = lambda k: gemm(a_q, blobs[k % R], y, M, N, K, workspace=ws)
        quant_us = run_timed(torch, lambda k: q4.q8_quantize(a, a_q), min(steps, 50), 5)["kernel_us"]
    elif s["kind"] == "gemv" and s.get("prepared"):
        prep = torch.empty(getattr(q4, f + "_gemv_prepare_bytes")(M, K), dtype=torch.uint8,
                           device="cuda")
        prepare = getattr(q4, f + "_gemv_prepare")
        prepare(a, M, K, prep)
        gemv = getattr(q4, f + "_gemv_prepared")
        fn = lambda k: gemv(prep, blobs[k % R], y, M, N, K)
        prep_us = run_timed(torch, lambda k: prepare(a, M, K, prep), min(steps, 50), 5)["kernel_us"]
    elif s["kind"] == "gemv" and s.get("splitk"):
        gemv = getattr(q4, f + "_gemv_splitk")
        ws_bytes = getattr(q4, f + "_gemv_splitk_workspace_bytes")(M, N, K, 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        fn = lambda k: gemv(a, blobs[k % R], y, M, N, K, 0, workspace=ws)
    elif s["kind"] == "gemv":
        gemv = getattr(q4, f + ("_gemv_bf16" if act == "bf16" else "_gemv"))
        fn = lambda k: gemv(a, blobs[k % R], y, M, N, K)
    else:
        entry = f + ("_gemm_bf16" if act == "bf16" else "_gemm_ws")
        gemm = getattr(q4, entry)
        ws_bytes = getattr(q4, entry.replace("_gemm_ws", "_gemm") + "_workspace_bytes")(M, N, K)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        fn = lambda k: gemm(a, blobs[k % R], y, M, N, K, workspace=ws)
    t = run_timed(torch, fn, steps, warmup)
    a_bytes = M * (K // 32) * 34 if act == "q8_0" else M * K * (2 if act == "bf16" else 4)
    algo_bytes = wbytes + a_bytes + M * N * 4
    flops = 2.0 * M * N * K
    kern_s = t["kernel_us"] * 1e-6
    row = {"workload": name, "format": fmt, "activations": act, "M": M, "N": N, "K": K,
           "weight_sha256": digest(blob), "activation_sha256": digest(a), "weight_copies": R,
           "cache": "cold" if R > 1 else "warm (one weight copy, MALL-resident)",
           "algorithmic_bytes": algo_bytes, "flops": flops, **t,
           "kernel_GBs": algo_bytes / kern_s / 1e9, "kernel_TFLOPs": flops / kern_s / 1e12,
           "job_GBs": algo_bytes * steps / t["wall_s"] / 1e9,
           "job_TFLOPs": flops * steps / t["wall_s"] / 1e12}
    if quant_us is not None:
        row["quantize_us"] = quant_us
        row["note"] = ("kernel_us is the product over Q8_0 activation blocks alone; quantizing "
                       "the f32 activations (q8_quantize, one more launch) takes quantize_us")
    if prep_us is not None:
        row["prepare_us"] = prep_us
        row["note"] = ("kernel_us is the GEMV from prepared operands alone; preparing them "
                       "(one more launch, shared by every weight matrix that multiplies the "
                       "same activations) takes prepare_us")
    if s["kind"] == "gemv":
        kernel = gemv_kernel_name(M, K, fmt, act, s.get("splitk", False), N, s.get("prepared"))
        row["roofline"] = hbm_roofline(algo_bytes, t["kernel_us"], name, kernel, "gemv")
        if s.get("splitk"):
            row["roofline"]["note"] = ("the time is the whole call: the split GEMV kernel plus "
                                       "the kernel that adds the splits' partials")
    else:
        kernel = gemm_kernel_name(K, fmt, act)
        if act == "q8_0":
            note = ("useful 2MNK flops over the dense f16 MFMA peak; the Q8_0 activations are "
                    "split into two binary16 terms, so 0.5 is this design's ceiling; the time is "
                    "the whole step (row-exponent and split kernels plus the GEMM kernel)")
        elif act == "bf16":
            note = ("useful 2MNK flops over the dense f16 MFMA peak; one binary16 term per "
                    "bfloat16 activation, so 1.0 is this design's ceiling; the time is the "
                    "whole step (row-exponent and operand kernels plus the GEMM kernel)")
        else:
            note = ("useful 2MNK flops over the dense f16 MFMA peak; the two-term activation "
                    "split issues 2 MFMA flops per useful flop, so 0.5 is this design's "
                    "ceiling; the time is the whole step (activation split kernel plus the "
                    "GEMM kernel)")
        row["roofline"] = {"bound": "mfma", "achieved": row["kernel_TFLOPs"],
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": row["kernel_TFLOPs"] / MFMA_F16_PEAK_TFLOPS,
                           "traffic": load_traffic(name, kernel, "gemm"), "kernel": kernel,
                           "note": note}
    row["kernel"] = kernel
    del blobs, blob, a, y
    torch.cuda.empty_cache()
    return row


def bench_dequant(torch, q4, wl, steps, warmup, name="dequant_14336x4096"):
    s = wl.WORKLOADS[name]
    N, K = s["N"], s["K"]
    fmt = s.get("fmt", "q4_0")
    blob = make_weight(torch, q4, wl, N, K, s["w_seed"], fmt)
    outs = [torch.empty(N * K, dtype=torch.float32, device="cuda") for _ in range(2)]
    dequant = getattr(q4, fmt[:2] + "_dequant")
    fn = lambda k: dequant(blob, outs[k % 2])
    t = run_timed(torch, fn, steps, warmup)
    algo = blob.numel() + N * K * 4
    kern_s = t["kernel_us"] * 1e-6
    kernel = "k_dequant<%s>" % FMT_TYPE[fmt]
    row = {"workload": name, "format": fmt, "kernel": kernel, "weight_sha256": digest(blob),
           "cache": "cold (%d MB per call)" % round(algo / 1e6), "algorithmic_bytes": algo, **t,
           "kernel_GBs": algo / kern_s / 1e9, "job_GBs": algo * steps / t["wall_s"] / 1e9}
    row["roofline"] = hbm_roofline(algo, t["kernel_us"], name, kernel, "dequant")
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
    fn = lambda k: q4.q8_quantize(xs[k % R], out)
    t = run_timed(torch, fn, steps, warmup)
    algo = n * 4 + n // 32 * 34
    kern_s = t["kernel_us"] * 1e-6
    row = {"workload": "quantize_2048x4096", "kernel": "k_quantize_q8_0", "input_copies": R,
           "input_sha256": digest(x),
           "cache": "cold", "algorithmic_bytes": algo, **t, "kernel_GBs": algo / kern_s / 1e9,
           "job_GBs": algo * steps / t["wall_s"] / 1e9}
    row["roofline"] = hbm_roofline(algo, t["kernel_us"], "quantize_2048x4096", "k_quantize_q8_0",
                                   "quantize")
    del xs, x, out
    torch.cuda.empty_cache()
    return row


def bench_stream_ceiling(torch, nbytes, steps, warmup, cold=True):
    """A plain 16-byte streaming read of `nbytes` (libq4probe.so) in the same
    harness and cache state as the GEMV rows: the practical ceiling for one
    launch that reads that much."""
    import ctypes
    path = os.path.join(ROOT, "block_quantized_weight_dequant_amd", "libq4probe.so")
    lib = ctypes.CDLL(path)
    lib.q4probe_stream_read.restype = ctypes.c_int
    lib.q4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
    R = copies_for_cold(nbytes) if cold else 1
    bufs = [torch.full((nbytes,), 0x37, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")

    def fn(k):
        st = lib.q4probe_stream_read(bufs[k % R].data_ptr(), nbytes, sink.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("q4probe_stream_read status %d" % st)

    t = run_timed(torch, fn, steps, warmup)
    row = {"workload": "stream_read_%dB" % nbytes, "kernel": "k_stream_read (libq4probe)",
           "copies": R, "cache": "cold" if R > 1 else "warm", "bytes": nbytes, **t,
           "kernel_GBs": nbytes / (t["kernel_us"] * 1e-6) / 1e9}
    row["frac_of_hbm_peak"] = row["kernel_GBs"] / HBM_PEAK_GBS
    del bufs, sink
    torch.cuda.empty_cache()
    return row


def copy_calibration(torch):
    """One 256 MiB device-to-device copy (read 256 MiB, write 256 MiB), for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 64 * 2 ** 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_each_way": n * 4, "launches": 3}


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
    # The other configurations the oracle can time in a few seconds: the same
    # decode GEMV on one core, the 8-row decode on all cores, and the
    # single-threaded dequant and quantize of the FFN-sized tensors.
    also = []

    def timed_reps(fn, budget):
        fn()
        n, t1 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el1 = time.perf_counter() - t1
            if el1 >= budget:
                return el1 / n
    t_one = timed_reps(lambda: oracle.q4_0_matmul(a, blob, N, K, threads=1), 2.0)
    also.append({"what": "1x4096x4096 decode GEMV", "value": algo / t_one / 1e9, "unit": "GB/s",
                 "cores": 1, "ms_each": 1e3 * t_one})
    s8 = wl.WORKLOADS["gemv_8x4096x4096"]
    a8 = wl.activations_f32(s8["a_seed"], s8["M"], K)
    t8 = timed_reps(lambda: oracle.q4_0_matmul(a8, blob, N, K, threads=threads), 1.0)
    also.append({"what": "8x4096x4096 decode GEMV", "value": (blob.size + a8.size * 4 + 8 * N * 4) / t8 / 1e9,
                 "unit": "GB/s", "cores": threads, "ms_each": 1e3 * t8})
    sd = wl.WORKLOADS["dequant_14336x4096"]
    wd = oracle.q4_0_quantize(wl.weights_f32(sd["w_seed"], sd["N"], sd["K"]))
    td = timed_reps(lambda: oracle.q4_0_dequant(wd), 0.5)
    also.append({"what": "dequant 14336x4096", "value": (wd.size + sd["N"] * sd["K"] * 4) / td / 1e9,
                 "unit": "GB/s", "cores": 1, "ms_each": 1e3 * td})
    sq = wl.WORKLOADS["quantize_2048x4096"]
    xq = wl.activations_f32(sq["x_seed"], sq["M"], sq["K"])
    tq = timed_reps(lambda: oracle.q8_0_quantize(xq), 0.5)
    also.append({"what": "Q8_0 quantize 2048x4096", "value": (xq.size * 4 + xq.size // 32 * 34) / tq / 1e9,
                 "unit": "GB/s", "cores": 1, "ms_each": 1e3 * tq})
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": algo * reps / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full 1x4096x4096 decode GEMVs in %.1f s (%.2f ms each), f64 sums"
                      % (reps, el, 1e3 * el / reps),
            "host": {"cpu_model": model, "logical_cpus": os.cpu_count(),
                     "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")},
            "also": also}


# -------------------------------------------------------------------- main

def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the sharding design is written up, not built); run with --gpus 1",
              file=sys.stderr)
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
        warm["roofline"]["traffic"] = None   # the counters were taken on the cold row
        rows.append(warm)
        log("row: dequant 14336x4096")
        rows.append(bench_dequant(torch, q4, wl, min(50, args.steps), min(args.warmup, 10)))
        log("row: Q8_0 quantize 2048x4096")
        rows.append(bench_quantize(torch, q4, wl, args.steps, args.warmup))
        # The tiny correctness configuration: 74 KB of weights, launch-dominated
        # (one weight copy; at this size the timed launches stay MALL-resident).
        log("row: gemv_1x256x512 (launch-dominated)")
        rows.append(bench_product(torch, q4, wl, "gemv_1x256x512", args.steps, args.warmup,
                                  cold=False))
        # The same path over Q8_0 weights.
        for name, st in (("q8_0_gemv_1x4096x4096", args.steps),
                         ("q8_0_gemv_8x4096x4096", args.steps),
                         ("q8_0_gemm_1024x4096x4096", 50), ("q8_0_gemm_2048x14336x4096", 20)):
            log("row: %s" % name)
            rows.append(bench_product(torch, q4, wl, name, min(st, args.steps),
                                      min(args.warmup, 10)))
        for name, st in (("gemv_bf16_1x4096x4096", args.steps),
                         ("gemv_bf16_8x4096x4096", args.steps),
                         ("q8_0_gemv_bf16_1x4096x4096", args.steps),
                         ("gemm_bf16_1024x4096x4096", 50), ("gemm_bf16_2048x14336x4096", 20),
                         ("q8_0_gemm_bf16_2048x14336x4096", 20)):
            log("row: %s" % name)
            rows.append(bench_product(torch, q4, wl, name, min(st, args.steps),
                                      min(args.warmup, 10)))
        for name, st in (("gemv_prepared_1x4096x4096", args.steps),
                         ("gemv_prepared_8x4096x4096", args.steps),
                         ("gemv_1x512x4096", args.steps), ("gemm_2048x1792x4096", 50),
                         ("gemv_1x512x14336", args.steps), ("gemv_splitk_1x512x14336", args.steps)):
            log("row: %s" % name)
            rows.append(bench_product(torch, q4, wl, name, min(st, args.steps),
                                      min(args.warmup, 10)))
        for name, st in (("gemv_q8a_1x4096x4096", args.steps), ("gemv_q8a_8x4096x4096", args.steps),
                         ("q8_0_gemv_q8a_1x4096x4096", args.steps),
                         ("gemm_q8a_1024x4096x4096", 50), ("gemm_q8a_2048x14336x4096", 20)):
            log("row: %s" % name)
            rows.append(bench_product(torch, q4, wl, name, min(st, args.steps),
                                      min(args.warmup, 10)))
        log("row: Q8_0 dequant 14336x4096")
        rows.append(bench_dequant(torch, q4, wl, min(50, args.steps), min(args.warmup, 10),
                                  "q8_0_dequant_14336x4096"))
    # Measured ceilings: a plain streaming read of the headline's bytes in the
    # same harness (cold), and of 1 GiB (the chip's sustained read rate).
    log("row: streaming-read ceilings")
    ceil = bench_stream_ceiling(torch, head["algorithmic_bytes"], args.steps, args.warmup)
    rows.append(ceil)
    if args.rows == "all":
        rows.append(bench_stream_ceiling(torch, 2 ** 30, 10, 3))
        # The quantize moves 42 MB; a streaming read of the same byte count in
        # the same harness bounds what a read-dominated kernel of that size gets.
        qrow = next(r for r in rows if r["workload"] == "quantize_2048x4096")
        qceil = bench_stream_ceiling(torch, qrow["algorithmic_bytes"], args.steps, args.warmup)
        rows.append(qceil)
        qrow["roofline"]["measured_read_ceiling_GBs"] = qceil["kernel_GBs"]
        qrow["roofline"]["frac_of_measured_read_ceiling"] = (
            qrow["roofline"]["achieved"] / qceil["kernel_GBs"])
        # The same for the 8-way shard of the decode GEMV.
        srow = next(r for r in rows if r["workload"] == "gemv_1x512x4096")
        sceil = bench_stream_ceiling(torch, srow["algorithmic_bytes"], args.steps, args.warmup)
        rows.append(sceil)
        srow["roofline"]["measured_read_ceiling_GBs"] = sceil["kernel_GBs"]
        srow["roofline"]["frac_of_measured_read_ceiling"] = (
            srow["roofline"]["achieved"] / sceil["kernel_GBs"])
        # And for the K = 14336 share, plain and split across workgroups.
        krows = [r for r in rows if r["workload"] in ("gemv_1x512x14336", "gemv_splitk_1x512x14336")]
        kceil = bench_stream_ceiling(torch, krows[0]["algorithmic_bytes"], args.steps, args.warmup)
        rows.append(kceil)
        for r in krows:
            r["roofline"]["measured_read_ceiling_GBs"] = kceil["kernel_GBs"]
            r["roofline"]["frac_of_measured_read_ceiling"] = r["roofline"]["achieved"] / kceil["kernel_GBs"]
    head["roofline"]["frac_of_measured_read_ceiling"] = (
        head["roofline"]["achieved"] / ceil["kernel_GBs"])
    head["roofline"]["measured_read_ceiling_GBs"] = ceil["kernel_GBs"]
    calib = copy_calibration(torch) if args.calibrate_copy else None

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cpu = cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": "Q4_0 GEMV GB/s (M=1, 4096²) + prefill GEMM TFLOP/s, % of roofline",
        "value": round(head["job_GBs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["wall_s"] * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 in/out; f16x2-split MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "gemv_1x4096x4096", "M": 1, "N": 4096, "K": 4096,
                   "cache": head["cache"], "weight_copies": head["weight_copies"],
                   "launch": head["launch"]},
        "roofline": {**head["roofline"], "kernel_us": head["kernel_us"]},
        "cpu_baseline": cpu,
        "rows": rows,
        "device": props.name,
        "device_arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "hip_runtime": torch.version.hip,
    }
    if calib:
        line["copy_calibration"] = calib
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
