"""CPU tests of the C ABI (include/q4.h): the library loads, exports exactly the
declared symbols, and rejects every invalid argument before launching anything.

No call here reaches a kernel launch: every argument set is invalid (or empty),
so the pointers, which are fake addresses or host buffers, are never touched.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")

binding = pytest.importorskip("block_quantized_weight_dequant_amd.binding")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The argument-check tests hand fake addresses to the library. Each call is
# invalid, so nothing is launched; as a second safeguard they do not run at all
# where a GPU is visible.
fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU-only test")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def _header_defines():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(Q4_\w+)\s+(\d+)", text)}


def test_exports_match_header():
    declared = _header_functions()
    assert declared == sorted(binding.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines()
                      if l.split()[-1].startswith(("q4_", "q8_")))
    assert exported == declared
    for name in declared:
        assert hasattr(binding.lib, name)


def test_probe_library_exports_its_header():
    # The measurement-only library: every function include/q4_probe.h
    # declares, and nothing else, is exported.
    hdr = os.path.join(ROOT, "include", "q4_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^\s*\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))
    lib = os.path.join(os.path.dirname(binding.LIB_PATH), "libq4probe.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("q4"))
    assert declared == exported == ["q4probe_stream_read", "q4probe_stream_read_cfg",
                                   "q4probe_stream_rw"]


def test_version_and_status_codes():
    defs = _header_defines()
    assert binding.q4_abi_version() == defs["Q4_ABI_VERSION"]
    for name in ("Q4_OK", "Q4_ERR_NULL", "Q4_ERR_SHAPE", "Q4_ERR_SIZE", "Q4_ERR_ALIGN",
                 "Q4_ERR_ALIAS", "Q4_ERR_LAUNCH", "Q4_ERR_WORKSPACE", "Q4_GEMV_MAX_ROWS",
                 "Q4_GEMM_SCRATCH_BYTES"):
        assert getattr(binding, name) == defs[name]
    strings = {binding.q4_status_string(c) for c in range(0, 8)}
    assert len(strings) == 8 and binding.q4_status_string(99) == "unknown status"


BASE = 0x7F0000000000       # fake, 16-byte aligned device-looking addresses
A, W, Y = BASE, BASE + (1 << 32), BASE + (2 << 32)


BLOCK_BYTES = {"q4": 18, "q8": 34}


def _prod(entry, a, w, wb, y, M, N, K):
    if entry.endswith(("_gemm_ws", "_gemm_bf16")):   # no workspace: these checks come before its own
        return binding.raw_status(entry, a, w, wb, y, M, N, K, 0, 0, 0)
    return binding.raw_status(entry, a, w, wb, y, M, N, K, 0)


def _wb(N, K, fmt="q4"):
    return N * (K // 32) * BLOCK_BYTES[fmt]


@fake_addresses
@pytest.mark.parametrize("entry", ["q4_gemv", "q4_gemm", "q4_gemm_ws", "q8_gemv", "q8_gemm",
                                   "q8_gemm_ws", "q4_gemm_bf16",
                                   "q8_gemm_bf16", "q4_gemv_bf16", "q8_gemv_bf16"])
def test_product_argument_checks(entry):
    S = binding
    f = entry[:2]
    wb = lambda N, K: _wb(N, K, f)
    # A blob of the other format's length is a size error.
    other = _wb(4, 64, "q8" if f == "q4" else "q4")
    assert _prod(entry, A, W, other, Y, 1, 4, 64) == S.Q4_ERR_SIZE
    assert _prod(entry, A, W, wb(4, 64), Y, 1, 4, 48) == S.Q4_ERR_SHAPE      # K % 32
    assert _prod(entry, A, W, 0, Y, 1, 4, 0) == S.Q4_ERR_SHAPE                # K < 32
    assert _prod(entry, A, W, wb(4, 64), Y, -1, 4, 64) == S.Q4_ERR_SHAPE
    assert _prod(entry, A, W, wb(4, 64), Y, 1, -4, 64) == S.Q4_ERR_SHAPE
    assert _prod(entry, A, W, wb(4, 64) + 1, Y, 1, 4, 64) == S.Q4_ERR_SIZE   # blob length
    assert _prod(entry, A, W, wb(4, 64) - BLOCK_BYTES[f], Y, 1, 4, 64) == S.Q4_ERR_SIZE
    assert _prod(entry, None, W, wb(4, 64), Y, 1, 4, 64) == S.Q4_ERR_NULL
    assert _prod(entry, A, None, wb(4, 64), Y, 1, 4, 64) == S.Q4_ERR_NULL
    assert _prod(entry, A, W, wb(4, 64), None, 1, 4, 64) == S.Q4_ERR_NULL
    assert _prod(entry, A + 4, W, wb(4, 64), Y, 1, 4, 64) == S.Q4_ERR_ALIGN
    assert _prod(entry, A, W + 2, wb(4, 64), Y, 1, 4, 64) == S.Q4_ERR_ALIGN
    assert _prod(entry, A, W, wb(4, 64), Y + 8, 1, 4, 64) == S.Q4_ERR_ALIGN
    assert _prod(entry, A, W, wb(4, 64), A + 128, 2, 4, 64) == S.Q4_ERR_ALIAS  # y inside a
    assert _prod(entry, A, W, wb(4, 64), W + 32, 1, 4, 64) == S.Q4_ERR_ALIAS   # y inside w
    assert _prod(entry, A, W, wb(8, 64), W - 16, 1, 8, 64) == S.Q4_ERR_ALIAS   # y ends inside w
    # empty problems: OK without looking at the pointers
    assert _prod(entry, None, None, wb(4, 64), None, 0, 4, 64) == S.Q4_OK
    assert _prod(entry, None, None, 0, None, 3, 0, 64) == S.Q4_OK


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_bf16_activations_are_two_bytes(f):
    # [2, 64] activations end 256 bytes (bfloat16) or 512 bytes (f32) after a:
    # an output at a + 256 overlaps the f32 form only. The bfloat16 call then
    # passes every product check and stops at its (missing) workspace.
    wb = _wb(4, 64, f)
    assert _prod(f + "_gemm_ws", A, W, wb, A + 256, 2, 4, 64) == binding.Q4_ERR_ALIAS
    assert _prod(f + "_gemm_bf16", A, W, wb, A + 256, 2, 4, 64) == binding.Q4_ERR_WORKSPACE
    assert _prod(f + "_gemm_bf16", A, W, wb, A + 240, 2, 4, 64) == binding.Q4_ERR_ALIAS
    assert _prod(f + "_gemv", A, W, wb, A + 256, 2, 4, 64) == binding.Q4_ERR_ALIAS
    assert _prod(f + "_gemv_bf16", A, W, wb, A + 240, 2, 4, 64) == binding.Q4_ERR_ALIAS


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
@pytest.mark.parametrize("act", ["", "_bf16"])
def test_gemv_row_limit(f, act):
    assert _prod(f + "_gemv" + act, A, W, _wb(4, 64, f), Y, 9, 4, 64) == binding.Q4_ERR_SHAPE
    assert _prod(f + "_gemv" + act, None, None, _wb(4, 64, f), None, 0, 4, 64) == binding.Q4_OK


@fake_addresses
def test_size_overflow():
    # 32-bit M, N, K cannot overflow a 64-bit byte count, but element counts can.
    assert binding.raw_status("q4_dequant", W, 18 * 2 ** 60, Y, 0, 0) == binding.Q4_ERR_SIZE
    assert binding.raw_status("q8_dequant", W, 34 * 2 ** 60, Y, 0, 0) == binding.Q4_ERR_SIZE
    assert binding.raw_status("q8_quantize", A, 2 ** 63, Y, 2 ** 58 * 34, 0) == binding.Q4_ERR_SIZE


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_dequant_argument_checks(f):
    S = binding
    b = BLOCK_BYTES[f]
    st = lambda w, wb, o, oe: binding.raw_status(f + "_dequant", w, wb, o, oe, 0)
    assert st(W, 2 * b - 1, Y, 64) == S.Q4_ERR_SIZE
    assert st(W, 2 * b, Y, 63) == S.Q4_ERR_SIZE
    assert st(W, 2 * BLOCK_BYTES["q4" if f == "q8" else "q8"], Y, 64) == S.Q4_ERR_SIZE
    assert st(None, 0, None, 0) == S.Q4_OK
    assert st(None, 2 * b, Y, 64) == S.Q4_ERR_NULL
    assert st(W, 2 * b, None, 64) == S.Q4_ERR_NULL
    assert st(W + 2, 2 * b, Y, 64) == S.Q4_ERR_ALIGN
    assert st(W, 2 * b, Y + 4, 64) == S.Q4_ERR_ALIGN
    assert st(W, 2 * b, W + 16, 64) == S.Q4_ERR_ALIAS
    assert st(W, 2 * b, W - 240, 64) == S.Q4_ERR_ALIAS


@fake_addresses
@pytest.mark.parametrize("entry,blk", [("q8_quantize", 34), ("q4_quantize", 18)])
def test_quantize_argument_checks(entry, blk):
    S = binding
    st = lambda x, n, o, ob: binding.raw_status(entry, x, n, o, ob, 0)
    assert st(A, 33, Y, blk) == S.Q4_ERR_SHAPE
    assert st(A, 64, Y, 2 * blk + 1) == S.Q4_ERR_SIZE
    assert st(A, 64, Y, blk) == S.Q4_ERR_SIZE
    assert st(None, 0, None, 0) == S.Q4_OK
    assert st(None, 64, Y, 2 * blk) == S.Q4_ERR_NULL
    assert st(A, 64, None, 2 * blk) == S.Q4_ERR_NULL
    assert st(A + 8, 64, Y, 2 * blk) == S.Q4_ERR_ALIGN
    assert st(A, 64, Y + 2, 2 * blk) == S.Q4_ERR_ALIGN
    assert st(A, 64, A + 128, 2 * blk) == S.Q4_ERR_ALIAS


def test_rejected_call_writes_nothing():
    # Host buffers stand in for device memory; a rejected call never reads or
    # writes them.
    y = np.full(64, 7.0, dtype=np.float32)
    a = np.ones(64, dtype=np.float32)
    w = np.zeros(4 * 18, dtype=np.uint8)
    st = binding.raw_status("q4_gemm_ws", a.ctypes.data, w.ctypes.data, w.size + 1, y.ctypes.data,
                            1, 2, 64, 0, 0, 0)
    assert st == binding.Q4_ERR_SIZE
    assert (y == 7.0).all()


@pytest.mark.parametrize("fn", ["q4_gemm_workspace_bytes", "q8_gemm_workspace_bytes"])
def test_gemm_workspace_bytes(fn):
    f = getattr(binding, fn)
    # Row exponents (int32, padded to 256 bytes), then the rows padded to whole
    # 128-row tiles, binary16 hi and lo per element.
    assert f(1, 1, 64) == 256 + 128 * 64 * 4
    assert f(128, 7, 4096) == 512 + 128 * 4096 * 4
    assert f(129, 7, 4096) == 768 + 256 * 4096 * 4
    assert f(1024, 4096, 4096) == 4096 + 1024 * 4096 * 4
    assert f(2 ** 31 - 1, 1, 2 ** 22) == 2 ** 33 + 2 ** 31 * 2 ** 22 * 4
    assert f(65536, 32767, 64) == 65536 * 4 + 65536 * 64 * 4
    # No split path (K % 64 != 0, K > 2^22, or M N >= 2^31: the general kernel):
    # the row exponents only.
    for M, N, K in [(5, 5, 96), (5, 5, 32), (5, 5, 4128), (5, 5, 2 ** 22 + 64), (5, 5, 2 ** 31 - 64),
                    (65536, 32768, 64), (2 ** 31 - 1, 2, 64)]:
        assert f(M, N, K) == ((M * 4 + 255) // 256) * 256, (M, N, K)
    # Empty or invalid shapes: no workspace.
    for M, N, K in [(0, 5, 64), (5, 0, 64), (-1, 5, 64), (5, -1, 64), (5, 5, 48), (5, 5, 0),
                    (5, 5, -64)]:
        assert f(M, N, K) == 0, (M, N, K)


@pytest.mark.parametrize("fn", ["q4_gemm_bf16_workspace_bytes", "q8_gemm_bf16_workspace_bytes"])
def test_gemm_bf16_workspace_bytes(fn):
    f = getattr(binding, fn)
    # Row exponents (int32, padded to 256 bytes), then one binary16 per element
    # of the 128-row-padded activations on the split path ...
    assert f(1, 1, 64) == 256 + 128 * 64 * 2
    assert f(64, 7, 4096) == 256 + 128 * 4096 * 2
    assert f(65, 7, 4096) == 512 + 128 * 4096 * 2
    assert f(2048, 14336, 4096) == 2048 * 4 + 2048 * 4096 * 2
    # ... else the f32 scaled activations: K % 64 != 0, or M N >= 2^31.
    assert f(5, 5, 96) == 256 + 5 * 96 * 4
    assert f(3, 9, 32) == 256 + 3 * 32 * 4
    assert f(65536, 32768, 64) == 65536 * 4 + 65536 * 64 * 4
    assert f(65536, 32767, 64) == 65536 * 4 + 65536 * 64 * 2
    assert f(3, 5, 2 ** 22 + 64) == 256 + 3 * (2 ** 22 + 64) * 4
    for M, N, K in [(0, 5, 64), (5, 0, 64), (-1, 5, 64), (5, -1, 64), (5, 5, 48), (5, 5, 0),
                    (5, 5, -64)]:
        assert f(M, N, K) == 0, (M, N, K)


@fake_addresses
@pytest.mark.parametrize("g", ["q4_gemm_ws", "q8_gemm_ws", "q4_gemm_bf16", "q8_gemm_bf16"])
@pytest.mark.parametrize("K", [64, 96])
def test_gemm_workspace_checks(g, K):
    S = binding
    f = g[:2]
    M, N = 3, 4
    need = getattr(binding, g.replace("_ws", "") + "_workspace_bytes")(M, N, K)
    assert need > 0   # every non-empty shape takes a workspace
    WS = BASE + (3 << 32)
    wbn = _wb(N, K, f)
    st = lambda ws, wsb: binding.raw_status(g, A, W, wbn, Y, M, N, K, ws, wsb, 0)
    assert st(WS, need - 1) == S.Q4_ERR_WORKSPACE
    assert st(None, 0) == S.Q4_ERR_WORKSPACE
    assert st(None, need) == S.Q4_ERR_NULL
    assert st(WS + 8, need) == S.Q4_ERR_ALIGN
    assert st(A + 16, need) == S.Q4_ERR_ALIAS                        # inside a
    assert st(W - need + 16, need) == S.Q4_ERR_ALIAS                 # ends inside w
    assert st(Y, need) == S.Q4_ERR_ALIAS                             # on y
    # Checks of a, w and y come first, and an empty problem needs nothing.
    assert binding.raw_status(g, A, W, wbn, Y, M, N, 48, None, 0, 0) == S.Q4_ERR_SHAPE
    assert binding.raw_status(g, None, None, wbn, None, 0, N, K, None, 0, 0) == S.Q4_OK


@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemv_splitk_workspace_bytes(f):
    ws = getattr(binding, f + "_gemv_splitk_workspace_bytes")
    # Auto: no split below 3 chunks per wavefront, else ceil(256 / (N/16)) splits,
    # at most K/32/64; each split a multiple of 8 blocks.
    assert ws(1, 512, 14336, 0) == 7 * 512 * 4          # 448 blocks (7 chunks): 8 wanted, 7 allowed
    assert ws(1, 512, 4096, 0) == 0                     # one 16-block chunk per wavefront
    assert ws(8, 1024, 8192, 0) == 0                    # two chunks per wavefront
    assert ws(1, 4096, 14336, 0) == 0                   # 256 column groups: no split
    assert ws(1, 64, 32768, 0) == 16 * 64 * 4           # 8 chunks, 4 groups: 64 wanted, 16 allowed
    assert ws(2, 1024, 32768, 0) == 4 * 2 * 1024 * 4    # 64 groups -> 4 splits
    # Requested splits, capped at one per 8 blocks and rounded to 8-block splits.
    assert ws(2, 300, 4096, 3) == 3 * 2 * 300 * 4       # 128 blocks -> 48, 48, 32
    assert ws(1, 64, 4096, 5) == 4 * 64 * 4             # ks = 26 rounded up to 32: 4 splits
    assert ws(1, 64, 256, 9) == 0                       # 8 blocks: one split at most
    assert ws(1, 64, 4096, 1) == 0
    # Off the streaming kernel (K % 256 != 0), invalid or empty: no workspace.
    for M, N, K, s in [(1, 64, 4128, 4), (0, 64, 4096, 2), (9, 64, 4096, 2), (1, 0, 4096, 2),
                       (1, 64, 4096, -1), (1, 64, 48, 2)]:
        assert ws(M, N, K, s) == 0, (M, N, K, s)


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemv_splitk_checks(f):
    S = binding
    wbn = _wb(64, 4096, f)
    st = lambda a, y, M, N, K, s, ws, wsb: binding.raw_status(f + "_gemv_splitk", a, W, wbn if N == 64 else _wb(N, K, f), y, M, N, K, s, ws, wsb, 0)
    need = getattr(binding, f + "_gemv_splitk_workspace_bytes")(1, 64, 4096, 4)
    assert need == 4 * 64 * 4
    WS = BASE + (3 << 32)
    assert st(A, Y, 9, 64, 4096, 4, WS, need) == S.Q4_ERR_SHAPE        # M > 8
    assert st(A, Y, 1, 64, 4096, -1, WS, need) == S.Q4_ERR_SHAPE       # negative splits
    assert st(A, Y, 1, 64, 4096, 4, WS, need - 4) == S.Q4_ERR_WORKSPACE
    assert st(A, Y, 1, 64, 4096, 4, None, need) == S.Q4_ERR_NULL
    assert st(A, Y, 1, 64, 4096, 4, WS + 4, need) == S.Q4_ERR_ALIGN
    assert st(A, Y, 1, 64, 4096, 4, Y, need) == S.Q4_ERR_ALIAS
    assert st(None, None, 0, 64, 4096, 4, None, 0) == S.Q4_OK          # empty


@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemv_prepare_bytes(f):
    pb = getattr(binding, f + "_gemv_prepare_bytes")
    # Two binary16 terms per activation (K/32 blocks x 4 lane groups x 2M rows x 16 B),
    # then M int32 exponents padded to 16 bytes.
    assert pb(1, 4096) == 128 * 4 * 2 * 16 + 16
    assert pb(8, 4096) == 128 * 4 * 16 * 16 + 32
    assert pb(5, 256) == 8 * 4 * 10 * 16 + 32
    for M, K in [(0, 4096), (9, 4096), (1, 4128), (1, 0), (1, -256), (-1, 256)]:
        assert pb(M, K) == 0, (M, K)


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemv_prepare_checks(f):
    S = binding
    need = getattr(binding, f + "_gemv_prepare_bytes")(2, 512)
    PR = BASE + (3 << 32)
    prep = lambda a, M, K, p, pb: binding.raw_status(f + "_gemv_prepare", a, M, K, p, pb, 0)
    assert prep(A, 9, 512, PR, need) == S.Q4_ERR_SHAPE
    assert prep(A, 2, 4128, PR, need) == S.Q4_ERR_SHAPE
    assert prep(A, 2, 512, PR, need - 1) == S.Q4_ERR_SIZE
    assert prep(None, 2, 512, PR, need) == S.Q4_ERR_NULL
    assert prep(A, 2, 512, PR + 8, need) == S.Q4_ERR_ALIGN
    assert prep(A, 2, 512, A + 16, need) == S.Q4_ERR_ALIAS
    assert prep(None, 0, 512, None, 0) == S.Q4_OK
    wbn = _wb(64, 512, f)
    run = lambda p, pb, w, wb, y, M, N, K: binding.raw_status(f + "_gemv_prepared", p, pb, w, wb, y, M, N, K, 0)
    assert run(PR, need, W, wbn, Y, 9, 64, 512) == S.Q4_ERR_SHAPE
    assert run(PR, need, W, _wb(64, 4128, f), Y, 2, 64, 4128) == S.Q4_ERR_SHAPE
    assert run(PR, need, W, wbn + 1, Y, 2, 64, 512) == S.Q4_ERR_SIZE
    assert run(PR, need - 16, W, wbn, Y, 2, 64, 512) == S.Q4_ERR_SIZE
    assert run(None, need, W, wbn, Y, 2, 64, 512) == S.Q4_ERR_NULL
    assert run(PR, need, W, wbn, Y + 4, 2, 64, 512) == S.Q4_ERR_ALIGN
    assert run(PR, need, W, wbn, PR + 32, 2, 64, 512) == S.Q4_ERR_ALIAS
    assert run(None, 0, None, wbn, None, 0, 64, 512) == S.Q4_OK


@fake_addresses
def test_binding_raises_q4error():
    with pytest.raises(binding.Q4Error) as e:
        binding.q4_gemm_ws(A, W, Y, 1, 4, 48, w_bytes=_wb(4, 64), stream=0, workspace=A + 4096,
                           workspace_bytes=4096)
    assert e.value.status == binding.Q4_ERR_SHAPE


def test_one_hip_runtime_in_process():
    # The binding loads PyTorch's HIP runtime before libq4.so, so both resolve
    # to one copy and PyTorch's stream handles are valid for the library.
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(runtimes) == 1, runtimes


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemv_q8a_checks(f):
    S = binding
    ab = lambda M, K: M * (K // 32) * 34
    st = lambda a, abn, w, wbn, y, M, N, K: binding.raw_status(f + "_gemv_q8a", a, abn, w, wbn,
                                                                y, M, N, K, 0)
    wb = _wb(4, 256, f)
    assert st(A, ab(9, 256), W, wb, Y, 9, 4, 256) == S.Q4_ERR_SHAPE        # M > 8
    assert st(A, ab(2, 256), W, wb, Y, 2, 4, 240) == S.Q4_ERR_SHAPE        # K % 32
    assert st(A, ab(2, 256), W, wb, Y, -1, 4, 256) == S.Q4_ERR_SHAPE
    assert st(A, ab(2, 256) - 34, W, wb, Y, 2, 4, 256) == S.Q4_ERR_SIZE   # activation blob
    assert st(A, 2 * 256 * 4, W, wb, Y, 2, 4, 256) == S.Q4_ERR_SIZE       # f32 length, not Q8_0
    assert st(A, ab(2, 256), W, wb + 1, Y, 2, 4, 256) == S.Q4_ERR_SIZE
    assert st(None, ab(2, 256), W, wb, Y, 2, 4, 256) == S.Q4_ERR_NULL
    assert st(A, ab(2, 256), W, wb, None, 2, 4, 256) == S.Q4_ERR_NULL
    assert st(A + 2, ab(2, 256), W, wb, Y, 2, 4, 256) == S.Q4_ERR_ALIGN
    assert st(A, ab(2, 256), W + 8, wb, Y, 2, 4, 256) == S.Q4_ERR_ALIGN
    assert st(A, ab(2, 256), W, wb, A + 16, 2, 4, 256) == S.Q4_ERR_ALIAS   # y inside a_q
    assert st(A, ab(2, 256), W, wb, W + 32, 2, 4, 256) == S.Q4_ERR_ALIAS   # y inside w
    assert st(None, 0, None, wb, None, 0, 4, 256) == S.Q4_OK                # empty
    assert st(None, ab(3, 256), None, 0, None, 3, 0, 256) == S.Q4_OK


@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemm_q8a_workspace_bytes(f):
    ws = getattr(binding, f + "_gemm_q8a_workspace_bytes")
    # Row exponents padded to 256 bytes, then two binary16 terms per element of
    # whole 128-row tiles on the split path (K % 64 == 0), else M K f32.
    assert ws(1024, 4096, 4096) == 4096 + 1024 * 4096 * 4
    assert ws(1, 64, 4096) == 256 + 128 * 4096 * 4
    assert ws(65, 64, 96) == 512 + 65 * 96 * 4
    assert ws(2, 64, 1 << 23) == 256 + 2 * (1 << 23) * 4           # K > 2^22: general kernel
    for M, N, K in [(0, 64, 4096), (1, 0, 4096), (1, 64, 48), (-1, 64, 4096)]:
        assert ws(M, N, K) == 0, (M, N, K)


@fake_addresses
@pytest.mark.parametrize("f", ["q4", "q8"])
def test_gemm_q8a_checks(f):
    S = binding
    M, N, K = 130, 4, 256
    ab = M * (K // 32) * 34
    wb = _wb(N, K, f)
    need = getattr(binding, f + "_gemm_q8a_workspace_bytes")(M, N, K)
    WS = BASE + (3 << 32)
    st = lambda a, abn, y, m, ws, wsb: binding.raw_status(f + "_gemm_q8a", a, abn, W, wb, y, m, N,
                                                          K, ws, wsb, 0)
    assert st(A, ab - 1, Y, M, WS, need) == S.Q4_ERR_SIZE
    assert st(A, M * K * 4, Y, M, WS, need) == S.Q4_ERR_SIZE            # f32 length
    assert st(A, ab, Y, -1, WS, need) == S.Q4_ERR_SHAPE
    assert st(None, ab, Y, M, WS, need) == S.Q4_ERR_NULL
    assert st(A + 2, ab, Y, M, WS, need) == S.Q4_ERR_ALIGN
    assert st(A, ab, A + 32, M, WS, need) == S.Q4_ERR_ALIAS              # y inside a_q
    assert st(A, ab, Y, M, WS, need - 1) == S.Q4_ERR_WORKSPACE
    assert st(A, ab, Y, M, None, need) == S.Q4_ERR_NULL
    assert st(A, ab, Y, M, WS + 8, need) == S.Q4_ERR_ALIGN
    assert st(A, ab, Y, M, A + 16, need) == S.Q4_ERR_ALIAS               # workspace over a_q
    assert st(A, ab, Y, M, Y, need) == S.Q4_ERR_ALIAS                    # workspace over y
    assert st(None, 0, None, 0, None, 0) == S.Q4_OK                      # empty


def test_host_tensors_are_refused_before_any_call():
    # A host tensor's data pointer would reach a kernel as a device address.
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        binding.q4_gemv(a, torch.zeros(4 * 2 * 18, dtype=torch.uint8), torch.zeros(16), 4, 4, 64)
    with pytest.raises(ValueError):
        binding.q8_quantize(torch.zeros(64), torch.zeros(68, dtype=torch.uint8))
