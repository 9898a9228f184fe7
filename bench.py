"""Benchmark of the Q4_0 (and Q8_0-weight) hot path on one MI355X.

Headline (the last stdout line's ``value``): the decode GEMV y[1, 4096] =
a[1, 4096] @ dequant(W[4096, 4096])^T, as whole-job GB/s of algorithmic
traffic (weight blocks + activations + output) over exactly K timed steps. One
step is one GEMV. The inputs are read cold: step k uses the (k mod R)-th of R
device copies of (weights, activations), and the R copies span more than
twice the 256 MiB last-level cache. All inputs are resident in HBM before
timing starts.

Timing: the K launches of a row are captured once into a HIP graph (plain
kernel nodes, no memset nodes), warmed up by replays, then replayed ``--reps``
times (default 5); each replay is bracketed by HIP events on the launch stream
and by torch.cuda.synchronize() on both sides. A launch's duration is a
replay's event-measured region divided by K (back-to-back launches, so it
includes the gap between kernels); a row reports the median, minimum and 90th
percentile of that over the replays, and ``value`` uses the host clock of the
median replay. Per-dispatch durations without the gaps come from the
rocprofv3 kernel trace (``profiles/``), keyed to rows by roctx ranges.

Every other row of the path is measured the same way: the 8-row GEMV, the
prefill GEMMs (1024 x 4096 x 4096 and 2048 x 14336 x 4096, through q4_gemm),
a warm-cache GEMV, the dequant of the 14336 x 4096 weight and the Q8_0
quantize of a 2048 x 4096 tensor; the same over Q8_0 weights; bfloat16 and
Q8_0-quantized activations; one GPU's share of an 8-way row split; and
streaming-read ceilings of the same byte counts. Each row is written to stderr
as one ``row: {json}`` line (and to ``--rows-out``); stdout ends with ONE
compact JSON line.

``roofline.traffic`` comes from the committed counter summary
profiles/traffic.json (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy of
known size) and is null when the kernel source has changed since; the GEMMs'
MFMA-busy fractions and the trace durations come from profiles/mfma_busy.json
and profiles/trace.json under the same rule.

The oracle (CPU, f64) is timed on this host's cores as ``cpu_baseline``: the
median of 5 runs of repeated full decode GEMVs, with the tiny and 8-row GEMVs,
one-core runs, 16 rows of the 1024 x 4096 x 4096 prefill GEMM (TFLOP/s) and
the dequant and quantize beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|headline]
    python bench.py --summarize --trace DIR [--fetch DIR --write DIR --mfma DIR]
        (no GPU: reads rocprofv3 output of profiled bench runs, writes profiles/)
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6      # MI355X dense f16 MFMA (no sparsity)
TWO_TERM_CEILING_TFLOPS = MFMA_F16_PEAK_TFLOPS / 2   # two f16 MFMA flops per useful flop
F32_VECTOR_PEAK_TFLOPS = 157.3     # MI355X f32 vector arithmetic
LLC_BYTES = 256 * 2 ** 20          # MI355X last-level (MALL) cache
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "gemv": "block_quantized_weight_dequant_amd/csrc/gemv.hip",
    "gemm": "block_quantized_weight_dequant_amd/csrc/gemm.hip",
    "dequant": "block_quantized_weight_dequant_amd/csrc/dequant.hip",
    "quantize": "block_quantized_weight_dequant_amd/csrc/quantize.hip",
    "probe": "block_quantized_weight_dequant_amd/csrc/probe/stream_read.hip",
}


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--reps", type=int, default=5, help="timed replays per row")
    p.add_argument("--rows", choices=["all", "headline"], default="all")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rows-out", help="write every row (and the CPU baseline's detail) here")
    p.add_argument("--spans-out", help="write each row's host-clock span here (for --summarize)")
    p.add_argument("--profile", action="store_true",
                   help="fixed warm-up (no time floor), for runs under rocprofv3")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run 256 MiB device copies (counter calibration)")
    p.add_argument("--summarize", action="store_true",
                   help="no GPU: summarize rocprofv3 output of profiled bench runs into profiles/")
    p.add_argument("--trace", help="rocprofv3 --kernel-trace --marker-trace output directory")
    p.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output directory")
    p.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output directory")
    p.add_argument("--mfma", help="rocprofv3 --pmc SQ_* output directory")
    p.add_argument("--out", default=PROFILES)
    p.add_argument("--probe-sweep", action="store_true",
                   help="sweep the streaming-read probe's launch shapes (no other rows)")
    p.add_argument("--sweep-out", help="write the sweep table here")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha256(kind):
    with open(os.path.join(ROOT, KERNEL_SOURCES[kind]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def kernel_kind(kernel):
    for key in ("gemv", "gemm", "dequant", "quantize"):
        if kernel.startswith("k_" + key) or kernel.startswith("k_row_exp") and key == "gemm":
            return key
    return "probe" if "stream_read" in kernel else None


def profile_record(fname, workload, kernel):
    """The committed per-workload record of `kernel` in profiles/<fname>, or None
    when absent or taken on a different kernel source."""
    try:
        with open(os.path.join(PROFILES, fname)) as f:
            rec = json.load(f)["workloads"].get(workload)
    except (OSError, ValueError, KeyError):
        return None
    if not rec or rec.get("kernel") != kernel:
        return None
    kind = kernel_kind(kernel)
    if kind is None or rec.get("source_sha256") != source_sha256(kind):
        return None
    return rec


def load_traffic(workload, kernel):
    rec = profile_record("traffic.json", workload, kernel)
    return rec.get("bytes_per_launch") if rec else None


def sig(x, n=4):
    """x rounded to n significant digits (for the compact line)."""
    if x is None or not isinstance(x, (int, float)) or x == 0 or not np.isfinite(x):
        return x
    return float("%.*g" % (n, x))


# ------------------------------------------------------------------ markers

class Marks:
    """roctx ranges around each row (seen by rocprofv3 --marker-trace; no-ops
    otherwise) and the same spans on the host clocks, for runs under
    rocprofv3 --pmc, which cannot record the markers."""

    def __init__(self):
        self.spans = []
        self.lib = None
        path = "/opt/rocm/lib/librocprofiler-sdk-roctx.so"
        if os.path.exists(path):
            try:
                lib = ctypes.CDLL(path)
                lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                lib.roctxRangePushA.restype = ctypes.c_int
                lib.roctxRangePop.restype = ctypes.c_int
                self.lib = lib
            except OSError:
                self.lib = None

    @staticmethod
    def _now():
        return {"boottime_ns": time.clock_gettime_ns(time.CLOCK_BOOTTIME),
                "monotonic_ns": time.clock_gettime_ns(time.CLOCK_MONOTONIC)}

    def push(self, name):
        if self.lib is not None:
            self.lib.roctxRangePushA(name.encode())
        self.spans.append({"name": name, "start": self._now()})

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()
        open_ = [s for s in self.spans if "end" not in s]
        open_[-1]["end"] = self._now()


MARKS = Marks()


# ----------------------------------------------------------------- timing

def run_timed(torch, fn, steps, warmup, reps, name, profile=False, min_warm_s=0.3):
    """Capture `steps` launches (fn(k), k = 0..steps-1) into one HIP graph, warm
    up by replaying it (>= warmup launches, and >= min_warm_s unless
    `profile`), then time `reps` replays, each with events on the current
    stream and the host clock, bracketed by synchronizations."""
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
    while done < warmup or (not profile and time.perf_counter() - t0 < min_warm_s):
        graph.replay()
        done += steps
        torch.cuda.synchronize()
    region_ms, wall_s = [], []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    MARKS.push(name + "/timed")
    for _ in range(reps):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        wall_s.append(time.perf_counter() - w0)
        region_ms.append(start.elapsed_time(end))
    MARKS.pop()
    del graph
    us = np.array(region_ms) * 1e3 / steps
    med = int(np.argsort(us)[len(us) // 2])
    return {"kernel_us": float(np.median(us)), "kernel_us_min": float(us.min()),
            "kernel_us_p90": float(np.percentile(us, 90)), "kernel_us_reps": [float(u) for u in us],
            "wall_s": wall_s[med], "region_ms": region_ms[med], "steps": steps, "reps": reps,
            "launch": "hip-graph replay of %d launches, %d timed replays" % (steps, reps)}


def copies_for_cold(nbytes):
    return max(2, int(np.ceil(2.2 * LLC_BYTES / max(nbytes, 1))))


def hbm_roofline(algo_bytes, kernel_us, workload, kernel):
    achieved = algo_bytes / (kernel_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(workload, kernel),
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


def quantize_kernel_name(n_blocks):
    """The Q8_0 quantizer instance the library launches for n_blocks blocks
    (mirrors launch_quant: two blocks per lane group while that still gives
    1024 workgroups, else one)."""
    return "k_quantize_q8_0<%d>" % (2 if -(-n_blocks // 64) >= 1024 else 1)


def gemv_kernel_name(M, K, fmt="q4_0", act="f32", splitk=False, N=0, prepared=False):
    """The kernel the library launches (mirrors launch_gemv_m, launch_gemv_q8a_m and
    gemv_split_plan)."""
    if act == "q8_0":
        if K % 256:
            return "k_gemv_q8a_any<%s, %d>" % (FMT_TYPE[fmt], M)
        groups = (N + 15) // 16
        la = K % 2048 == 0   # whole-line weight loads (and then non-temporal ones)
        LA = "true" if la else "false"
        if M > 1 and groups > 256 and K // 32 in (64, 128):   # row-group loops
            return "k_gemv_q8a<%s, %d, 8, %d, %s, true, %s>" % (
                FMT_TYPE[fmt], M, K // 256, "true" if (la or fmt == "q4_0") else "false", LA)
        if groups <= 256 and K // 32 == 64:   # one 8-block chunk per wavefront
            return "k_gemv_q8a<%s, %d, 8, 8, true, false, %s>" % (FMT_TYPE[fmt], M, LA)
        ch16 = (K // 32) % 16 == 0 and (groups <= 256 or M == 1)
        nt = la or (ch16 and groups <= 256 and K // 32 <= 128)   # non-temporal weight loads
        return "k_gemv_q8a<%s, %d, 8, %d, %s, false, %s>" % (FMT_TYPE[fmt], M, 16 if ch16 else 8,
                                                            "true" if nt else "false", LA)
    bf = "true" if act == "bf16" else "false"
    if K % 256:
        return "k_gemv<%s, %d, %s>" % (FMT_TYPE[fmt], M, bf)
    nblk = K // 32
    # Whole-line weight loads where every row is a whole number of 128-byte
    # lines (the bench's buffers are line-aligned); with them every launch
    # takes non-temporal loads.
    la = K % 2048 == 0
    LA = "true" if la else "false"
    tf = lambda b: "true" if b else "false"
    if prepared:
        ch = 16 if nblk % 16 == 0 else 8
        if (N + 15) // 16 > 256 and nblk in (64, 128):   # row-group loops
            return "k_gemv_stream<%s, %d, 8, %d, false, 2, 16, %s, true, %s>" % (
                FMT_TYPE[fmt], M, nblk // 8, tf(la), LA)
        if nblk == 64:   # one 8-block chunk per wavefront
            return "k_gemv_stream<%s, %d, 8, 8, false, 2, 16, true, false, %s>" % (FMT_TYPE[fmt], M, LA)
        nt = la or ((N + 15) // 16 <= 256 and nblk <= 8 * ch)
        return "k_gemv_stream<%s, %d, 8, %d, false, 2, 16, %s, false, %s>" % (FMT_TYPE[fmt], M, ch,
                                                                              tf(nt), LA)
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
    if M == 1 and splits == 1 and ch == 16 and (N + 15) // 16 <= 128 and ks <= 8 * ch:
        return "k_gemv_stream<%s, 1, 8, 16, %s, 1, 8, true, false, %s>" % (FMT_TYPE[fmt], bf, LA)   # eight rows per workgroup
    if splits == 1 and ((ch == 16 and ks == 8 * 16) or ks == 8 * 8) and (N + 15) // 16 > 256:
        return "k_gemv_stream<%s, %d, 8, %d, %s, 0, 16, %s, true, %s>" % (   # row-group loops
            FMT_TYPE[fmt], M, ks // 8, bf, tf(la or M > 1), LA)
    if splits == 1 and ks == 8 * 8:   # one 8-block chunk per wavefront
        return "k_gemv_stream<%s, %d, 8, 8, %s, 0, 16, true, false, %s>" % (FMT_TYPE[fmt], M, bf, LA)
    spread = (N + 15) // 16 * splits > 256 or ks > 8 * ch   # non-temporal loads otherwise
    al = spread and not (ch == 16 and ni > 8)
    return "k_gemv_stream<%s, %d, 8, %d, %s, %d, 16, %s, false, %s>" % (
        FMT_TYPE[fmt], M, ch, bf, 1 if al else 0, tf(la or not spread), LA)


def gemm_kernel_name(K, fmt="q4_0", act="f32"):
    if K % 64:
        return "k_gemm_any<%s>" % FMT_TYPE[fmt]
    return "k_gemm_split<%s, %s>" % (FMT_TYPE[fmt], "true" if act == "bf16" else "false")


GEMM_NOTES = {
    "f32": ("useful 2MNK flops; the two-term activation split issues 2 MFMA flops per useful "
            "flop, so frac_two_term_ceiling is against half the dense f16 peak; the time is the "
            "whole step (row-exponent, split and GEMM kernels, through q4_gemm)"),
    "q8_0": ("useful 2MNK flops; the Q8_0 activations are split into two binary16 terms (half "
             "the dense f16 peak is this design's ceiling); the time is the whole step "
             "(row-exponent, split and GEMM kernels)"),
    "bf16": ("useful 2MNK flops; one binary16 term per bfloat16 activation, so the dense f16 "
             "peak is this design's ceiling; the time is the whole step (row-exponent, operand "
             "and GEMM kernels)"),
}


def bench_product(torch, q4, wl, name, steps, warmup, reps, profile, cold=True, label=None):
    label = label or name
    s = wl.WORKLOADS[name]
    M, N, K = s["M"], s["N"], s["K"]
    fmt = s.get("fmt", "q4_0")
    f = fmt[:2]
    act = s.get("act", "f32")
    MARKS.push(label)
    blob = make_weight(torch, q4, wl, N, K, s["w_seed"], fmt)
    if act == "bf16":
        a = torch.from_numpy(wl.activations_bf16(s["a_seed"], M, K).view("int16")).cuda()
    else:
        a = torch.from_numpy(wl.activations_f32(s["a_seed"], M, K)).cuda()
    y = torch.empty(M * N, dtype=torch.float32, device="cuda")
    wbytes = blob.numel()
    a_dev_bytes = a.numel() * a.element_size()
    # Cold rows rotate R sets of (weights, activations) that together exceed the
    # last-level cache twice; the prepared GEMV rotates its weights only.
    R = (copies_for_cold(wbytes) if s.get("prepared") else copies_for_cold(wbytes + a_dev_bytes)) \
        if cold else 1
    blobs = [blob] + [blob.clone() for _ in range(R - 1)]
    acts = [a] + ([a.clone() for _ in range(R - 1)] if not s.get("prepared") else [])
    A = lambda k: acts[k % len(acts)]
    prep_us = quant_us = None
    if act == "q8_0":
        # The activations are quantized once per set, outside the timed region
        # (its own time is quantize_us); the product reads the Q8_0 blocks.
        aqs = []
        for x in acts:
            aq = torch.empty(M * (K // 32) * 34, dtype=torch.uint8, device="cuda")
            q4.q8_quantize(x, aq)
            aqs.append(aq)
        if s["kind"] == "gemv":
            gemv = getattr(q4, f + "_gemv_q8a")
            fn = lambda k: gemv(aqs[k % R], blobs[k % R], y, M, N, K)
        else:
            gemm = getattr(q4, f + "_gemm_q8a")
            ws = torch.empty(max(getattr(q4, f + "_gemm_q8a_workspace_bytes")(M, N, K), 16),
                             dtype=torch.uint8, device="cuda")
            fn = lambda k: gemm(aqs[k % R], blobs[k % R], y, M, N, K, workspace=ws)
        quant_us = run_timed(torch, lambda k: q4.q8_quantize(acts[0], aqs[0]), min(steps, 50), 5,
                             1, label + "/quantize", profile)["kernel_us"]
    elif s["kind"] == "gemv" and s.get("prepared"):
        prep = torch.empty(getattr(q4, f + "_gemv_prepare_bytes")(M, K), dtype=torch.uint8,
                           device="cuda")
        prepare = getattr(q4, f + "_gemv_prepare")
        prepare(a, M, K, prep)
        gemv = getattr(q4, f + "_gemv_prepared")
        fn = lambda k: gemv(prep, blobs[k % R], y, M, N, K)
        prep_us = run_timed(torch, lambda k: prepare(a, M, K, prep), min(steps, 50), 5, 1,
                            label + "/prepare", profile)["kernel_us"]
    elif s["kind"] == "gemv" and s.get("splitk"):
        gemv = getattr(q4, f + "_gemv_splitk")
        ws_bytes = getattr(q4, f + "_gemv_splitk_workspace_bytes")(M, N, K, 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        fn = lambda k: gemv(A(k), blobs[k % R], y, M, N, K, 0, workspace=ws)
    elif s["kind"] == "gemv":
        gemv = getattr(q4, f + ("_gemv_bf16" if act == "bf16" else "_gemv"))
        fn = lambda k: gemv(A(k), blobs[k % R], y, M, N, K)
    elif act == "bf16":
        gemm = getattr(q4, f + "_gemm_bf16")
        ws = torch.empty(max(getattr(q4, f + "_gemm_bf16_workspace_bytes")(M, N, K), 16),
                         dtype=torch.uint8, device="cuda")
        fn = lambda k: gemm(A(k), blobs[k % R], y, M, N, K, workspace=ws)
    else:
        # The f32 GEMM through the entry with the pages' argument list (its
        # scratch is the library's; its results equal q4_gemm_ws's).
        gemm = getattr(q4, f + "_gemm")
        fn = lambda k: gemm(A(k), blobs[k % R], y, M, N, K)
    t = run_timed(torch, fn, steps, warmup, reps, label, profile)
    MARKS.pop()
    a_bytes = M * (K // 32) * 34 if act == "q8_0" else M * K * (2 if act == "bf16" else 4)
    algo_bytes = wbytes + a_bytes + M * N * 4
    flops = 2.0 * M * N * K
    kern_s = t["kernel_us"] * 1e-6
    row = {"workload": label, "format": fmt, "activations": act, "M": M, "N": N, "K": K,
           "weight_sha256": digest(blob), "activation_sha256": digest(a), "input_sets": R,
           "cache": "cold" if R > 1 else "warm (one set of inputs, MALL-resident)",
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
        row["roofline"] = hbm_roofline(algo_bytes, t["kernel_us"], name, kernel)
        if s.get("splitk"):
            row["roofline"]["note"] = ("the time is the whole call: the split GEMV kernel plus "
                                       "the kernel that adds the splits' partials")
    else:
        kernel = gemm_kernel_name(K, fmt, act)
        peak = MFMA_F16_PEAK_TFLOPS if act == "bf16" else TWO_TERM_CEILING_TFLOPS
        busy = profile_record("mfma_busy.json", name, kernel)
        row["roofline"] = {"bound": "mfma", "achieved": row["kernel_TFLOPs"], "peak": peak,
                           "unit": "TFLOP/s", "frac": row["kernel_TFLOPs"] / peak,
                           "frac_f16_dense": row["kernel_TFLOPs"] / MFMA_F16_PEAK_TFLOPS,
                           "traffic": load_traffic(name, kernel), "kernel": kernel,
                           "mfma_busy": busy.get("mfma_busy") if busy else None,
                           "note": GEMM_NOTES[act]}
    row["kernel"] = kernel
    del blobs, blob, acts, a, y
    torch.cuda.empty_cache()
    return row


def bench_dequant(torch, q4, wl, steps, warmup, reps, profile, name="dequant_14336x4096"):
    s = wl.WORKLOADS[name]
    N, K = s["N"], s["K"]
    fmt = s.get("fmt", "q4_0")
    MARKS.push(name)
    blob = make_weight(torch, q4, wl, N, K, s["w_seed"], fmt)
    outs = [torch.empty(N * K, dtype=torch.float32, device="cuda") for _ in range(2)]
    dequant = getattr(q4, fmt[:2] + "_dequant")
    fn = lambda k: dequant(blob, outs[k % 2])
    t = run_timed(torch, fn, steps, warmup, reps, name, profile)
    MARKS.pop()
    algo = blob.numel() + N * K * 4
    kern_s = t["kernel_us"] * 1e-6
    kernel = "k_dequant<%s>" % FMT_TYPE[fmt]
    row = {"workload": name, "format": fmt, "kernel": kernel, "weight_sha256": digest(blob),
           "cache": "cold (%d MB per call)" % round(algo / 1e6), "algorithmic_bytes": algo, **t,
           "kernel_GBs": algo / kern_s / 1e9, "job_GBs": algo * steps / t["wall_s"] / 1e9}
    row["roofline"] = hbm_roofline(algo, t["kernel_us"], name, kernel)
    del blob, outs
    torch.cuda.empty_cache()
    return row


def bench_quantize(torch, q4, wl, steps, warmup, reps, profile):
    name = "quantize_2048x4096"
    s = wl.WORKLOADS[name]
    n = s["M"] * s["K"]
    MARKS.push(name)
    x = torch.from_numpy(wl.activations_f32(s["x_seed"], s["M"], s["K"])).cuda().reshape(-1)
    R = copies_for_cold(n * 4)
    xs = [x] + [x.clone() for _ in range(R - 1)]
    out = torch.empty(n // 32 * 34, dtype=torch.uint8, device="cuda")
    fn = lambda k: q4.q8_quantize(xs[k % R], out)
    t = run_timed(torch, fn, steps, warmup, reps, name, profile)
    MARKS.pop()
    algo = n * 4 + n // 32 * 34
    kern_s = t["kernel_us"] * 1e-6
    kernel = quantize_kernel_name(n // 32)
    row = {"workload": name, "kernel": kernel, "input_sets": R,
           "input_sha256": digest(x),
           "cache": "cold", "algorithmic_bytes": algo, **t, "kernel_GBs": algo / kern_s / 1e9,
           "job_GBs": algo * steps / t["wall_s"] / 1e9}
    row["roofline"] = hbm_roofline(algo, t["kernel_us"], name, kernel)
    del xs, x, out
    torch.cuda.empty_cache()
    return row


def bench_stream_ceiling(torch, nbytes, steps, warmup, reps, profile, cold=True):
    """A plain 16-byte streaming read of `nbytes` (libq4probe.so) in the same
    harness and cache state as the GEMV rows: the practical ceiling for one
    launch that reads that much."""
    path = os.path.join(ROOT, "block_quantized_weight_dequant_amd", "libq4probe.so")
    lib = ctypes.CDLL(path)
    lib.q4probe_stream_read.restype = ctypes.c_int
    lib.q4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
    name = "stream_read_%dB" % nbytes
    MARKS.push(name)
    R = copies_for_cold(nbytes) if cold else 1
    bufs = [torch.full((nbytes,), 0x37, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")

    def fn(k):
        st = lib.q4probe_stream_read(bufs[k % R].data_ptr(), nbytes, sink.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("q4probe_stream_read status %d" % st)

    t = run_timed(torch, fn, steps, warmup, reps, name, profile)
    MARKS.pop()
    row = {"workload": name, "kernel": "k_stream_read (libq4probe)",
           "copies": R, "cache": "cold" if R > 1 else "warm", "bytes": nbytes, **t,
           "kernel_GBs": nbytes / (t["kernel_us"] * 1e-6) / 1e9}
    row["frac_of_hbm_peak"] = row["kernel_GBs"] / HBM_PEAK_GBS
    del bufs, sink
    torch.cuda.empty_cache()
    return row


def bench_rw_ceiling(torch, groups, read_words, write_words, steps, warmup, reps, profile):
    """Reading groups * read_words and writing groups * write_words 16-byte
    words, interleaved in that proportion (q4probe_stream_rw), cold: the
    ceiling for one launch that turns that many input bytes into that many
    output bytes (the quantizer 64 : 17, the dequant 9 : 64)."""
    path = os.path.join(ROOT, "block_quantized_weight_dequant_amd", "libq4probe.so")
    lib = ctypes.CDLL(path)
    lib.q4probe_stream_rw.restype = ctypes.c_int
    lib.q4probe_stream_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    rb, wb = groups * read_words * 16, groups * write_words * 16
    name = "stream_rw_%dB_%dB" % (rb, wb)
    MARKS.push(name)
    R = copies_for_cold(rb + wb)
    srcs = [torch.full((rb,), 0x37, dtype=torch.uint8, device="cuda") for _ in range(R)]
    dsts = [torch.empty(wb, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")

    # The fastest of the probe's shapes (groups per wavefront, cached or
    # non-temporal loads and stores) is the ceiling.
    best = None
    for loads in (1, 2, 4, 8):
        for flags in range(4):
            def fn(k, loads=loads, flags=flags):
                st = lib.q4probe_stream_rw(srcs[k % R].data_ptr(), dsts[k % R].data_ptr(), groups,
                                           read_words, write_words, loads, flags, sink.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
                if st != 0:
                    raise RuntimeError("q4probe_stream_rw status %d" % st)

            t = run_timed(torch, fn, steps, warmup, reps, "%s/l%d_f%d" % (name, loads, flags),
                          profile)
            t["loads"], t["flags"] = loads, flags
            if best is None or t["kernel_us"] < best["kernel_us"]:
                best = t
    t = best
    MARKS.pop()
    row = {"workload": name, "kernel": "k_stream_rw<%d, %s, %s> (libq4probe)" % (
               t["loads"], "true" if t["flags"] & 1 else "false",
               "true" if t["flags"] & 2 else "false"), "copies": R,
           "cache": "cold", "read_bytes": rb, "write_bytes": wb, **t,
           "kernel_GBs": (rb + wb) / (t["kernel_us"] * 1e-6) / 1e9}
    row["frac_of_hbm_peak"] = row["kernel_GBs"] / HBM_PEAK_GBS
    del srcs, dsts, sink
    torch.cuda.empty_cache()
    return row


def probe_sweep(torch, sizes, steps, warmup, reps, out_path=None):
    """The streaming read (libq4probe) of each size, cold, over every launch
    shape q4probe_stream_read_cfg offers: threads per workgroup x loads per
    thread x plain / non-temporal loads x grid-strided / blocked. The fastest shape at a size is the
    practical ceiling of one launch that reads that many bytes."""
    path = os.path.join(ROOT, "block_quantized_weight_dequant_amd", "libq4probe.so")
    lib = ctypes.CDLL(path)
    lib.q4probe_stream_read_cfg.restype = ctypes.c_int
    lib.q4probe_stream_read_cfg.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]
    lines, best = [], {}
    for nbytes in sizes:
        R = copies_for_cold(nbytes)
        bufs = [torch.full((nbytes,), 0x37, dtype=torch.uint8, device="cuda") for _ in range(R)]
        sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
        lines.append("")
        lines.append("%d bytes, cold (%d copies), %d launches per replay, median of %d replays"
                     % (nbytes, R, steps, reps))
        lines.append("%8s %6s %4s %4s %9s %10s %10s %8s" % ("threads", "loads", "nt", "blk",
                                                             "grid", "us", "GB/s", "frac"))
        for nt, blk in ((0, 0), (1, 0), (0, 1), (1, 1)):
            for T in (64, 128, 256, 512, 1024):
                for L in (1, 2, 4, 8, 16):
                    n16 = nbytes // 16
                    grid = -(-n16 // (T * L))

                    def fn(k, T=T, L=L, fl=nt | (blk << 1)):
                        st = lib.q4probe_stream_read_cfg(bufs[k % R].data_ptr(), nbytes,
                                                         sink.data_ptr(), T, L, fl,
                                                         torch.cuda.current_stream().cuda_stream)
                        if st != 0:
                            raise RuntimeError("q4probe_stream_read_cfg status %d" % st)

                    t = run_timed(torch, fn, steps, warmup, reps,
                                  "sweep_%dB_t%d_l%d_nt%d_b%d" % (nbytes, T, L, nt, blk), True)
                    gbs = nbytes / (t["kernel_us"] * 1e-6) / 1e9
                    lines.append("%8d %6d %4d %4d %9d %10.3f %10.1f %8.3f" % (
                        T, L, nt, blk, grid, t["kernel_us"], gbs, gbs / HBM_PEAK_GBS))
                    if nbytes not in best or t["kernel_us"] < best[nbytes]["us"]:
                        best[nbytes] = {"threads": T, "loads": L, "nontemporal": nt,
                                        "blocked": blk, "grid": grid, "us": t["kernel_us"],
                                        "GBs": gbs}
        lines.append("best: %s" % json.dumps(best[nbytes]))
        del bufs, sink
        torch.cuda.empty_cache()
    text = ["Streaming-read ceiling: q4probe_stream_read_cfg over its launch shapes (one MI355X, "
            "gfx950)", "",
            "command: python3 bench.py --probe-sweep --steps %d --warmup %d --reps %d" % (
                steps, warmup, reps)] + lines
    if out_path:
        with open(out_path, "w") as f:
            f.write("\n".join(text) + "\n")
    for l in text:
        log(l)
    return best


def copy_calibration(torch):
    """Three 256 MiB device-to-device copies (each reads 256 MiB and writes
    256 MiB), for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 64 * 2 ** 20
    MARKS.push("copy_calibration")
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    MARKS.push("copy_calibration/timed")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    MARKS.pop()
    MARKS.pop()
    return {"copy_bytes_each_way": n * 4, "launches": 3}


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(wl):
    """The oracle (plain C, f64 sums, OpenMP over outputs) on this host. Each
    figure is the median of 5 runs; a run repeats the call until its share of
    time has passed. Headline: full 1 x 4096 x 4096 decode GEMVs on all cores."""
    import oracle
    threads = oracle.max_threads()

    def median_rate(call, nbytes, run_s):
        call()                                   # warm
        rates, calls = [], 0
        for _ in range(5):
            n, t1 = 0, time.perf_counter()
            while True:
                call()
                n += 1
                el = time.perf_counter() - t1
                if el >= run_s:
                    break
            rates.append(nbytes * n / el / 1e9)
            calls += n
        return float(np.median(rates)), calls

    def gemv_case(wname, cores, run_s):
        s = wl.WORKLOADS[wname]
        M, N, K = s["M"], s["N"], s["K"]
        blob = oracle.q4_0_quantize(wl.weights_f32(s["w_seed"], N, K))
        a = wl.activations_f32(s["a_seed"], M, K)
        nbytes = blob.size + M * K * 4 + M * N * 4
        rate, calls = median_rate(lambda: oracle.q4_0_matmul(a, blob, N, K, threads=cores),
                                  nbytes, run_s)
        return {"what": wname, "value": rate, "unit": "GB/s", "cores": cores,
                "ms_each": nbytes / rate / 1e6, "calls": calls}

    def gemm_case(wname, rows, cores, run_s):
        # The first `rows` activation rows of the GEMM against its whole
        # weight: the same per-output work as the full product, in TFLOP/s.
        s = wl.WORKLOADS[wname]
        N, K = s["N"], s["K"]
        blob = oracle.q4_0_quantize(wl.weights_f32(s["w_seed"], N, K))
        a = wl.activations_f32(s["a_seed"], s["M"], K)[:rows]
        flops = 2.0 * rows * N * K
        rate, calls = median_rate(lambda: oracle.q4_0_matmul(a, blob, N, K, threads=cores),
                                  flops / 1e3, run_s)
        return {"what": "%s (first %d rows)" % (wname, rows), "value": rate, "unit": "TFLOP/s",
                "cores": cores, "ms_each": flops / (rate * 1e12) * 1e3, "calls": calls}

    head = gemv_case("gemv_1x4096x4096", threads, 1.0)
    also = [gemv_case("gemv_1x256x512", threads, 0.2), gemv_case("gemv_1x4096x4096", 1, 1.0),
            gemv_case("gemv_8x4096x4096", threads, 1.0), gemv_case("gemv_8x4096x4096", 1, 0.6)]
    gemm = gemm_case("gemm_1024x4096x4096", 16, threads, 1.0)
    also.append(gemm)
    sd = wl.WORKLOADS["dequant_14336x4096"]
    wd = oracle.q4_0_quantize(wl.weights_f32(sd["w_seed"], sd["N"], sd["K"]))
    nb = wd.size + sd["N"] * sd["K"] * 4
    rate, calls = median_rate(lambda: oracle.q4_0_dequant(wd), nb, 0.3)
    also.append({"what": "dequant_14336x4096", "value": rate, "unit": "GB/s", "cores": 1,
                 "ms_each": nb / rate / 1e6, "calls": calls})
    sq = wl.WORKLOADS["quantize_2048x4096"]
    xq = wl.activations_f32(sq["x_seed"], sq["M"], sq["K"])
    nb = xq.size * 4 + xq.size // 32 * 34
    rate, calls = median_rate(lambda: oracle.q8_0_quantize(xq), nb, 0.3)
    also.append({"what": "quantize_2048x4096", "value": rate, "unit": "GB/s", "cores": 1,
                 "ms_each": nb / rate / 1e6, "calls": calls})
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": head["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": ("median of 5 runs of ~1 s of full 1x4096x4096 decode GEMVs (%d calls, "
                       "%.2f ms each), f64 sums" % (head["calls"], head["ms_each"])),
            "host": {"cpu_model": model, "logical_cpus": os.cpu_count(),
                     "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")},
            "also": also}


# ------------------------------------------------------------ the rows

GEMV_ROWS = ["gemv_8x4096x4096"]
GEMM_ROWS = ["gemm_1024x4096x4096", "gemm_2048x14336x4096"]
MORE_ROWS = [
    ("q8_0_gemv_1x4096x4096", None), ("q8_0_gemv_8x4096x4096", None),
    ("q8_0_gemm_1024x4096x4096", 50), ("q8_0_gemm_2048x14336x4096", 20),
    ("gemv_bf16_1x4096x4096", None), ("gemv_bf16_8x4096x4096", None),
    ("q8_0_gemv_bf16_1x4096x4096", None), ("gemm_bf16_1024x4096x4096", 50),
    ("gemm_bf16_2048x14336x4096", 20), ("q8_0_gemm_bf16_2048x14336x4096", 20),
    ("gemv_prepared_1x4096x4096", None), ("gemv_prepared_8x4096x4096", None),
    ("gemv_8x14336x4096", None),
    ("gemv_1x512x4096", None), ("gemm_2048x1792x4096", 50), ("gemv_1x512x14336", None),
    ("gemv_splitk_1x512x14336", None), ("gemv_q8a_1x4096x4096", None),
    ("gemv_q8a_8x4096x4096", None), ("q8_0_gemv_q8a_1x4096x4096", None),
    ("gemm_q8a_1024x4096x4096", 50), ("gemm_q8a_2048x14336x4096", 20),
]
GEMM_STEPS = {"gemm_1024x4096x4096": 50, "gemm_2048x14336x4096": 20}


def emit_row(row, rows):
    rows.append(row)
    log("row: " + json.dumps(row))


def compact_gemm(row):
    r = row["roofline"]
    return {"us": sig(row["kernel_us"]), "TFLOPs": sig(row["kernel_TFLOPs"]),
            "frac_f16_dense": sig(r["frac_f16_dense"], 3), "frac_two_term_ceiling": sig(r["frac"], 3),
            "mfma_busy": sig(r["mfma_busy"], 3)}


def compact_hbm(row):
    return {"us": sig(row["kernel_us"]), "GBs": sig(row["kernel_GBs"]),
            "frac": sig(row["roofline"]["frac"], 3)}


def main_bench(args):
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
    S, W, P, reps = args.steps, args.warmup, args.profile, args.reps
    small_w = min(W, 10)
    if args.probe_sweep:
        best = probe_sweep(torch, [9469952, 42467328], S, W, reps, args.sweep_out)
        print(json.dumps({"probe_sweep_best": best}), flush=True)
        return

    log("headline: decode GEMV 1x4096x4096, cold inputs")
    head = bench_product(torch, q4, wl, "gemv_1x4096x4096", S, W, reps, P)
    rows = []
    emit_row(head, rows)
    log("ceiling: streaming read of the headline's bytes")
    ceil = bench_stream_ceiling(torch, head["algorithmic_bytes"], S, W, reps, P)
    head["roofline"]["measured_read_ceiling_GBs"] = ceil["kernel_GBs"]
    head["roofline"]["frac_of_measured_read_ceiling"] = head["roofline"]["achieved"] / ceil["kernel_GBs"]
    emit_row(ceil, rows)
    by = {}
    if args.rows == "all":
        for name in GEMV_ROWS:
            by[name] = bench_product(torch, q4, wl, name, S, small_w, reps, P)
            emit_row(by[name], rows)
        for name in GEMM_ROWS:
            by[name] = bench_product(torch, q4, wl, name, min(GEMM_STEPS[name], S), small_w, reps, P)
            emit_row(by[name], rows)
        warm = bench_product(torch, q4, wl, "gemv_1x4096x4096", S, W, reps, P, cold=False,
                             label="gemv_1x4096x4096_warm")
        emit_row(warm, rows)
        by["dequant"] = bench_dequant(torch, q4, wl, min(50, S), small_w, reps, P)
        emit_row(by["dequant"], rows)
        by["quantize"] = bench_quantize(torch, q4, wl, S, W, reps, P)
        emit_row(by["quantize"], rows)
        qceil = bench_stream_ceiling(torch, by["quantize"]["algorithmic_bytes"], S, W, reps, P)
        by["quantize"]["roofline"]["measured_read_ceiling_GBs"] = qceil["kernel_GBs"]
        by["quantize"]["roofline"]["frac_of_measured_read_ceiling"] = (
            by["quantize"]["roofline"]["achieved"] / qceil["kernel_GBs"])
        emit_row(qceil, rows)
        # Read-and-write ceilings in each kernel's own proportion (eight blocks a
        # group: 1024 bytes in, 272 out for the quantizer; 144 in, 1024 out for
        # the dequant).
        for key, nblocks, a_w, b_w in (("quantize", 2048 * 4096 // 32, 64, 17),
                                       ("dequant", 14336 * 4096 // 32, 9, 64)):
            c = bench_rw_ceiling(torch, nblocks // 8, a_w, b_w, min(50, S), small_w, reps, P)
            by[key]["roofline"]["measured_rw_ceiling_GBs"] = c["kernel_GBs"]
            by[key]["roofline"]["frac_of_measured_rw_ceiling"] = (
                by[key]["roofline"]["achieved"] / c["kernel_GBs"])
            emit_row(c, rows)
        # The tiny correctness configuration: 74 KB of weights, launch-dominated
        # (one set of inputs; at this size the timed launches stay MALL-resident).
        emit_row(bench_product(torch, q4, wl, "gemv_1x256x512", S, W, reps, P, cold=False), rows)
        for name, st in MORE_ROWS:
            r = bench_product(torch, q4, wl, name, min(st or S, S), small_w, reps, P)
            if name in ("gemv_1x512x4096", "gemv_1x512x14336", "gemv_splitk_1x512x14336",
                        "gemv_8x14336x4096"):
                c = bench_stream_ceiling(torch, r["algorithmic_bytes"], S, W, reps, P)
                r["roofline"]["measured_read_ceiling_GBs"] = c["kernel_GBs"]
                r["roofline"]["frac_of_measured_read_ceiling"] = r["roofline"]["achieved"] / c["kernel_GBs"]
                if name != "gemv_splitk_1x512x14336":
                    emit_row(c, rows)
            by[name] = r
            emit_row(r, rows)
        emit_row(bench_dequant(torch, q4, wl, min(50, S), small_w, reps, P,
                               "q8_0_dequant_14336x4096"), rows)
        emit_row(bench_stream_ceiling(torch, 2 ** 30, min(10, S), 3, reps, P), rows)
    if args.calibrate_copy:
        copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        cpu = cpu_baseline(wl)
        log("row: " + json.dumps({"workload": "cpu_baseline", **cpu}))

    if args.rows_out:
        with open(args.rows_out, "w") as f:
            json.dump({"rows": rows, "cpu_baseline": cpu}, f, indent=1)
    if args.spans_out:
        with open(args.spans_out, "w") as f:
            json.dump({"spans": MARKS.spans}, f, indent=1)

    hr = head["roofline"]
    trace = profile_record("trace.json", "gemv_1x4096x4096", hr["kernel"])
    line = {
        "metric": "Q4_0 GEMV GB/s (M=1, 4096²) + prefill GEMM TFLOP/s, % of roofline",
        "value": sig(head["job_GBs"], 5),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": sig(head["wall_s"] * 1e3 / S, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gemv_1x4096x4096", "M": 1, "N": 4096, "K": 4096, "weights": "Q4_0",
                   "cache": "cold", "input_sets": head["input_sets"],
                   "compute": "binary16 hi/lo split on MFMA, f32 accumulate"},
        "roofline": {"bound": "hbm", "achieved": sig(hr["achieved"]), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": sig(hr["frac"], 4), "traffic": hr["traffic"],
                     "kernel": hr["kernel"], "kernel_us": sig(head["kernel_us"]),
                     "kernel_us_min": sig(head["kernel_us_min"]),
                     "kernel_us_p90": sig(head["kernel_us_p90"]),
                     "trace_us_mean": sig(trace.get("mean_us")) if trace else None,
                     "measured_read_ceiling_GBs": sig(hr["measured_read_ceiling_GBs"]),
                     "frac_of_measured_read_ceiling": sig(hr["frac_of_measured_read_ceiling"], 3)},
    }
    if by:
        line["gemv_8x4096x4096"] = compact_hbm(by["gemv_8x4096x4096"])
        # Eight rows sit near the ridge of HBM and f32 vector arithmetic, so
        # the useful FLOP rate is given against the chip's f32 vector peak too.
        c3 = by["gemv_8x4096x4096"]
        line["gemv_8x4096x4096"]["TFLOPs"] = sig(c3["kernel_TFLOPs"], 3)
        line["gemv_8x4096x4096"]["frac_f32_vector_peak"] = sig(c3["kernel_TFLOPs"] / F32_VECTOR_PEAK_TFLOPS, 3)
        line["gemm"] = {"1024x4096x4096": compact_gemm(by["gemm_1024x4096x4096"]),
                        "2048x14336x4096": compact_gemm(by["gemm_2048x14336x4096"])}
        line["dequant_14336x4096"] = compact_hbm(by["dequant"])
        line["quantize_2048x4096"] = compact_hbm(by["quantize"])
        for key, lk in (("dequant", "dequant_14336x4096"), ("quantize", "quantize_2048x4096")):
            fr = by[key]["roofline"].get("frac_of_measured_rw_ceiling")
            if fr is not None:
                line[lk]["frac_of_rw_ceiling"] = sig(fr, 3)
    if cpu:
        line["cpu_baseline"] = {"value": sig(cpu["value"]), "unit": "GB/s", "cores": cpu["cores"],
                                "kind": "oracle",
                                "sample": "median of 5 ~1 s runs of full 1x4096x4096 GEMVs (f64)",
                                "cpu": cpu["host"]["cpu_model"][:40]}
        g = next((x for x in cpu["also"] if x["unit"] == "TFLOP/s"), None)
        if g:
            line["cpu_baseline"]["gemm"] = {"what": g["what"], "value": sig(g["value"], 3),
                                            "unit": "TFLOP/s", "cores": g["cores"]}
    line["device"] = "%s %s, %d CUs" % (props.name, getattr(props, "gcnArchName", ""),
                                        props.multi_processor_count)
    print(json.dumps(line, ensure_ascii=False), flush=True)


# ------------------------------------------------- profile summaries (no GPU)

def _read_csv(directory, suffix):
    paths = []
    for base, _, files in os.walk(directory):
        paths += [os.path.join(base, f) for f in files if f.endswith(suffix)]
    rows = []
    for p in sorted(paths):
        with open(p, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _short_kernel(name):
    """'void q4k::k_gemv_stream<q4k::FmtQ4_0, 1, 8, 16, false, 0>(...)' ->
    'k_gemv_stream<FmtQ4_0, 1, 8, 16, false, 0>'."""
    n = name.replace("(anonymous namespace)::", "").split("(")[0]
    return n.replace("void ", "").replace("q4k::", "").replace("q4probe::", "").strip()


def _spans(directory):
    """Row spans of a profiled bench run: the roctx ranges of its marker trace
    if present, else the host-clock spans the run wrote (spans.json)."""
    marks = _read_csv(directory, "marker_api_trace.csv")
    out = {}
    if marks:
        for m in marks:
            out.setdefault(m["Function"], []).append((int(m["Start_Timestamp"]),
                                                      int(m["End_Timestamp"])))
        return out, "roctx"
    with open(os.path.join(directory, "spans.json")) as f:
        spans = json.load(f)["spans"]
    for s in spans:
        out.setdefault(s["name"], []).append((s["start"]["boottime_ns"], s["end"]["boottime_ns"]))
    return out, "host CLOCK_BOOTTIME"


def _in(spans, t):
    return any(a <= t <= b for a, b in spans)


def _timed_rows(spans):
    """{workload: [spans]} for the timed part of every row."""
    return {k[:-len("/timed")]: v for k, v in spans.items() if k.endswith("/timed")}


def summarize_trace(directory):
    spans, how = _spans(directory)
    timed = _timed_rows(spans)
    disp = _read_csv(directory, "kernel_trace.csv")
    per = {}
    for d in disp:
        t0, t1 = int(d["Start_Timestamp"]), int(d["End_Timestamp"])
        for wname, sp in timed.items():
            if _in(sp, t0):
                per.setdefault(wname, {}).setdefault(_short_kernel(d["Kernel_Name"]), []).append(
                    (t1 - t0) / 1e3)
    return per, how


def summarize(args):
    os.makedirs(args.out, exist_ok=True)
    shas = {k: source_sha256(k) for k in KERNEL_SOURCES}
    cmd_note = ("python3 bench.py --summarize --trace <trace> --fetch <fetch> --write <write> "
                "--mfma <mfma>")
    if args.trace:
        per, how = summarize_trace(args.trace)
        recs, lines = {}, []
        lines.append("Per-dispatch kernel durations by bench row, from rocprofv3 kernel traces "
                     "(one MI355X, gfx950)")
        lines.append("")
        lines.append("command (trace):")
        lines.append("  cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --marker-trace "
                     "--stats --output-format csv -d <trace> -o trace -- python3 <repo>/bench.py "
                     "--profile --no-cpu-baseline --steps 20 --warmup 5")
        lines.append("summary: " + cmd_note)
        lines.append("rows: dispatches inside each row's timed replays (%s ranges)" % how)
        lines.append("")
        lines.append("%-34s %-48s %6s %9s %9s %9s %9s" % ("workload", "kernel", "n", "mean_us",
                                                         "median_us", "min_us", "p90_us"))
        for wname in per:
            for kern, durs in sorted(per[wname].items(), key=lambda kv: -sum(kv[1])):
                a = np.array(durs)
                rec = {"kernel": kern, "count": int(a.size), "mean_us": float(a.mean()),
                       "median_us": float(np.median(a)), "min_us": float(a.min()),
                       "p90_us": float(np.percentile(a, 90))}
                kind = kernel_kind(kern)
                if kind:
                    rec["source_sha256"] = shas[kind]
                lines.append("%-34s %-48s %6d %9.3f %9.3f %9.3f %9.3f" % (
                    wname, kern[:48], a.size, rec["mean_us"], rec["median_us"], rec["min_us"],
                    rec["p90_us"]))
                # The row's main kernel is the longest-running one.
                if wname not in recs:
                    recs[wname] = rec
        with open(os.path.join(args.out, "kernel_trace_by_workload.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        with open(os.path.join(args.out, "trace.json"), "w") as f:
            json.dump({"workloads": recs}, f, indent=1)
        stats = _read_csv(args.trace, "kernel_stats.csv")
        if stats:
            out = ["rocprofv3 --stats of the same traced run (all dispatches, warm-up included; "
                   "one MI355X, gfx950)", "",
                   "%-60s %7s %11s %10s %10s %10s" % ("kernel", "calls", "total_us", "mean_us",
                                                      "min_us", "max_us")]
            for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
                out.append("%-60s %7s %11.1f %10.3f %10.3f %10.3f" % (
                    _short_kernel(r["Name"])[:60], r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                    float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
            with open(os.path.join(args.out, "kernel_stats_bench.txt"), "w") as f:
                f.write("\n".join(out) + "\n")
        log("wrote kernel_trace_by_workload.txt, kernel_stats_bench.txt and trace.json (%d rows)"
            % len(recs))
    if args.fetch and args.write:
        summarize_traffic(args, shas)
    if args.mfma:
        summarize_mfma(args, shas)


def _counter_rows(directory):
    """{workload: {kernel: {counter: [value per dispatch]}}} of a --pmc run,
    dispatches assigned to rows by the run's host-clock spans (a counter's
    records of one dispatch are summed)."""
    spans, _ = _spans(directory)
    timed = _timed_rows(spans)
    acc = {}
    for d in _read_csv(directory, "counter_collection.csv"):
        t0 = int(d["Start_Timestamp"])
        for wname, sp in timed.items():
            if _in(sp, t0):
                per = acc.setdefault(wname, {}).setdefault(_short_kernel(d["Kernel_Name"]), {})
                by_dispatch = per.setdefault(d["Counter_Name"], {})
                did = d["Dispatch_Id"]
                by_dispatch[did] = by_dispatch.get(did, 0.0) + float(d["Counter_Value"])
    return {w: {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in ks.items()}
            for w, ks in acc.items()}


def _main_kernel(kernels, trace_recs, wname):
    if wname in trace_recs:
        return trace_recs[wname]["kernel"]
    return max(kernels, key=lambda k: len(next(iter(kernels[k].values()))))


def summarize_traffic(args, shas):
    fetch = _counter_rows(args.fetch)
    write = _counter_rows(args.write)
    try:
        with open(os.path.join(args.out, "trace.json")) as f:
            trace_recs = json.load(f)["workloads"]
    except OSError:
        trace_recs = {}
    # Calibration: the 256 MiB copies (read 2^28 and write 2^28 bytes each).
    cf = fetch.get("copy_calibration", {})
    cw = write.get("copy_calibration", {})
    fk = np.mean([v for k in cf.values() for v in k.get("FETCH_SIZE", [])])
    wk = np.mean([v for k in cw.values() for v in k.get("WRITE_SIZE", [])])
    fscale, wscale = 2 ** 18 / fk, 2 ** 18 / wk          # KiB copied / KiB counted
    from block_quantized_weight_dequant_amd import workloads as wl
    recs, lines = {}, []
    lines += ["HBM traffic per launch from rocprofv3 counters (one MI355X, gfx950)", "",
              "commands (two passes, one counter each):",
              "  cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d "
              "<fetch> -o fetch -- python3 <repo>/bench.py --profile --no-cpu-baseline --steps 20 "
              "--warmup 5 --calibrate-copy --spans-out <fetch>/spans.json",
              "  (the same with WRITE_SIZE into <write>)",
              "summary: python3 bench.py --summarize --trace <trace> --fetch <fetch> --write <write>",
              "",
              "calibration: three 256 MiB device-to-device copies in the same run",
              "  FETCH_SIZE read %.1f KiB per copy for 262144 KiB copied -> reads scale x %.4f"
              % (fk, fscale),
              "  WRITE_SIZE read %.1f KiB per copy for 262144 KiB copied -> writes scale x %.4f"
              % (wk, wscale), "",
              "%-32s %-46s %12s %12s %14s %8s" % ("workload", "kernel", "read_B", "write_B",
                                                  "algorithmic_B", "ratio")]
    for wname in fetch:
        if wname == "copy_calibration" or wname not in write:
            continue
        kern = _main_kernel(fetch[wname], trace_recs, wname)
        if kern not in fetch[wname] or kern not in write[wname]:
            continue
        rd = float(np.mean(fetch[wname][kern]["FETCH_SIZE"])) * 1024 * fscale
        wr = float(np.mean(write[wname][kern]["WRITE_SIZE"])) * 1024 * wscale
        algo = _algorithmic_bytes(wl, wname)
        kind = kernel_kind(kern)
        recs[wname] = {"kernel": kern, "source_sha256": shas.get(kind), "read_bytes_per_launch": round(rd),
                       "write_bytes_per_launch": round(wr), "bytes_per_launch": round(rd + wr),
                       "algorithmic_bytes": algo}
        lines.append("%-32s %-46s %12d %12d %14s %8s" % (
            wname, kern[:46], rd, wr, algo if algo else "-",
            "%.3f" % ((rd + wr) / algo) if algo else "-"))
    with open(os.path.join(args.out, "hbm_traffic_by_workload.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(args.out, "traffic.json"), "w") as f:
        json.dump({"calibration": {"fetch_scale": fscale, "write_scale": wscale},
                   "workloads": recs}, f, indent=1)
    log("wrote hbm_traffic_by_workload.txt and traffic.json (%d rows)" % len(recs))


def _algorithmic_bytes(wl, wname):
    """Algorithmic bytes of one launch of a workload (for the traffic ratio);
    None for rows that are not a product, dequant or quantize."""
    base = wname.replace("_warm", "")
    s = wl.WORKLOADS.get(base)
    if s is None:
        return None
    if s["kind"] == "quantize":
        n = s["M"] * s["K"]
        return n * 4 + n // 32 * 34
    bb = BLOCK_BYTES[s.get("fmt", "q4_0")]
    w = s["N"] * (s["K"] // 32) * bb
    if s["kind"] == "dequant":
        return w + s["N"] * s["K"] * 4
    act = s.get("act", "f32")
    a = s["M"] * (s["K"] // 32) * 34 if act == "q8_0" else s["M"] * s["K"] * (2 if act == "bf16" else 4)
    return w + a + s["M"] * s["N"] * 4


def summarize_mfma(args, shas):
    rows = _counter_rows(args.mfma)
    try:
        with open(os.path.join(args.out, "trace.json")) as f:
            trace_recs = json.load(f)["workloads"]
    except OSError:
        trace_recs = {}
    recs, lines = {}, []
    lines += ["MFMA utilisation of the GEMM kernels from rocprofv3 counters (one MI355X, gfx950)", "",
              "command:",
              "  cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
              "SQ_BUSY_CU_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU --output-format csv -d <mfma> -o mfma "
              "-- python3 <repo>/bench.py --profile --no-cpu-baseline --steps 20 --warmup 5 "
              "--spans-out <mfma>/spans.json",
              "summary: python3 bench.py --summarize --trace <trace> --mfma <mfma>", "",
              "mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CU_CYCLES x 4 SIMDs): the share of "
              "the kernel's busy SIMD cycles the matrix cores were busy; VALU/MFMA = "
              "SQ_INSTS_VALU / SQ_INSTS_MFMA", "",
              "%-32s %-32s %10s %12s %9s %8s" % ("workload", "kernel", "mfma_busy", "INSTS_MFMA",
                                                "VALU/MFMA", "n")]
    for wname, ks in rows.items():
        if not wname.startswith("gemm") and "_gemm" not in wname:
            continue
        kern = _main_kernel(ks, trace_recs, wname)
        c = ks.get(kern, {})
        if not all(x in c for x in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
                                    "SQ_INSTS_MFMA", "SQ_INSTS_VALU")):
            continue
        busy = float(np.mean(c["SQ_VALU_MFMA_BUSY_CYCLES"]))
        cu = float(np.mean(c["SQ_BUSY_CU_CYCLES"]))
        mf = float(np.mean(c["SQ_INSTS_MFMA"]))
        va = float(np.mean(c["SQ_INSTS_VALU"]))
        if not mf or not cu:
            continue   # not a matrix-core kernel (e.g. the activations' quantize)
        frac = busy / (cu * 4)
        recs[wname] = {"kernel": kern, "source_sha256": shas.get(kernel_kind(kern)),
                       "mfma_busy": frac, "valu_per_mfma": va / mf if mf else None,
                       "insts_mfma": mf}
        lines.append("%-32s %-32s %10.3f %12d %9.2f %8d" % (
            wname, kern[:32], frac, mf, recs[wname]["valu_per_mfma"],
            len(c["SQ_INSTS_MFMA"])))
    with open(os.path.join(args.out, "gemm_mfma_busy_by_workload.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(args.out, "mfma_busy.json"), "w") as f:
        json.dump({"workloads": recs}, f, indent=1)
    log("wrote gemm_mfma_busy_by_workload.txt and mfma_busy.json (%d rows)" % len(recs))


def main():
    args = parse_args()
    if args.summarize:
        summarize(args)
        return
    main_bench(args)


if __name__ == "__main__":
    main()
