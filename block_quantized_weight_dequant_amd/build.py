"""Build libq4.so, the gfx950 HIP library behind include/q4.h, and the
measurement-only libq4probe.so (include/q4_probe.h), in this package directory
(in-tree, so they travel with the source tree).

    python -m block_quantized_weight_dequant_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq4.so")
PROBE_LIB = os.path.join(PKG, "libq4probe.so")

SOURCES = ["abi.cpp", "validate.cpp", "dequant.hip", "quantize.hip", "gemv.hip", "gemm.hip"]
PROBE_SOURCES = ["probe/stream_read.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled for every kernel: the compiler would
# otherwise form v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          "--offload-arch=" + ARCH, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0].replace("/", "_") + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip"] + cmd[1:]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), proc.stdout, proc.stderr))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (proc.stdout, proc.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
