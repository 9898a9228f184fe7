"""Seeded random shapes through every product entry point, both weight formats
and every activation type, against the oracle's f64 products (sections
qmatvec_q4_0 and matmul_q4_0_tiled of "fuel-vulkan-kernels — quantized (GGML)
kernel contracts"; the activation types as in their own tests). K is drawn
among multiples of 32 (so every kernel path is reached: K % 256 == 0 or not,
K % 64 == 0 or not), M and N are ragged against the 16- and 128-row tiles, and
every output must meet |y - y_ref| <= 1e-5 * sum|a w| + 1e-6."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import Guarded, assert_within_tolerance, to_dev, weight_blob  # noqa: E402

KINDS = ["gemv", "gemm_ws", "gemv_bf16", "gemm_bf16", "gemv_q8a", "gemm_q8a", "gemv_splitk", "gemm"]


def _case(i):
    r = np.random.default_rng(9000 + i)
    kind = KINDS[i % len(KINDS)]
    fmt = "q4_0" if (i // len(KINDS)) % 2 == 0 else "q8_0"
    K = 32 * int(r.choice([1, 2, 3, 5, 8, 9, 16, 24, 40, 64, 96, 128, 129]))
    if kind.startswith("gemv"):
        M = int(r.integers(1, 9))
        N = int(r.integers(1, 700))
    else:
        M = int(r.integers(1, 300))
        N = int(r.integers(1, 400))
    while M * N * K > 60_000_000:
        N = max(1, N // 2)
    return kind, fmt, M, N, K


@pytest.mark.parametrize("i", range(64))
def test_random_shape(i):
    kind, fmt, M, N, K = _case(i)
    f = fmt[:2]
    blob = weight_blob(fmt, N, K, 9100 + i)
    w = to_dev(blob)
    y = Guarded(M * N, torch.float32)
    a32 = wl.activations_f32(9200 + i, M, K)
    if kind.endswith("bf16"):
        bits = wl.activations_bf16(9200 + i, M, K)
        getattr(binding, "%s_%s" % (f, kind))(to_dev(bits.view(np.int16)), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul")(oracle.bf16_to_f32(bits), blob, N, K)
    elif kind.endswith("q8a"):
        a_q = oracle.q8_0_quantize(a32)
        getattr(binding, "%s_%s" % (f, kind))(to_dev(a_q), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul_q8a")(a_q, M, blob, N, K)
    elif kind == "gemv_splitk":
        getattr(binding, f + "_gemv_splitk")(to_dev(a32), w, y.view, M, N, K, 0)
        ref, bound = getattr(oracle, fmt + "_matmul")(a32, blob, N, K)
    else:
        getattr(binding, "%s_%s" % (f, kind))(to_dev(a32), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul")(a32, blob, N, K)
    torch.cuda.synchronize()
    assert y.guards_intact()
    assert_within_tolerance(y.host().reshape(M, N), ref, bound,
                            "%s %s %dx%dx%d" % (kind, fmt, M, N, K))


WIDE_KINDS = ["gemv", "gemv_bf16", "gemv_q8a", "gemv_prepared"]


def _wide_case(i):
    # More row groups than compute units at K = 2048 or 4096 (one chunk per
    # wavefront), where the GEMVs walk the row groups, with ragged N.
    r = np.random.default_rng(9500 + i)
    kind = WIDE_KINDS[i % len(WIDE_KINDS)]
    fmt = "q4_0" if (i // len(WIDE_KINDS)) % 2 == 0 else "q8_0"
    K = int(r.choice([2048, 4096]))
    M = int(r.integers(1, 9))
    N = int(r.integers(4097, 20001))
    return kind, fmt, M, N, K


@pytest.mark.parametrize("i", range(24))
def test_random_wide_gemv(i):
    kind, fmt, M, N, K = _wide_case(i)
    f = fmt[:2]
    blob = weight_blob(fmt, N, K, 9600 + i)
    w = to_dev(blob)
    y = Guarded(M * N, torch.float32)
    a32 = wl.activations_f32(9700 + i, M, K)
    if kind == "gemv_bf16":
        bits = wl.activations_bf16(9700 + i, M, K)
        getattr(binding, f + "_gemv_bf16")(to_dev(bits.view(np.int16)), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul")(oracle.bf16_to_f32(bits), blob, N, K)
    elif kind == "gemv_q8a":
        a_q = oracle.q8_0_quantize(a32)
        getattr(binding, f + "_gemv_q8a")(to_dev(a_q), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul_q8a")(a_q, M, blob, N, K)
    elif kind == "gemv_prepared":
        prep = torch.empty(getattr(binding, f + "_gemv_prepare_bytes")(M, K), dtype=torch.uint8,
                           device="cuda")
        getattr(binding, f + "_gemv_prepare")(to_dev(a32), M, K, prep)
        getattr(binding, f + "_gemv_prepared")(prep, w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul")(a32, blob, N, K)
    else:
        getattr(binding, f + "_gemv")(to_dev(a32), w, y.view, M, N, K)
        ref, bound = getattr(oracle, fmt + "_matmul")(a32, blob, N, K)
    torch.cuda.synchronize()
    assert y.guards_intact()
    assert_within_tolerance(y.host().reshape(M, N), ref, bound,
                            "%s %s %dx%dx%d" % (kind, fmt, M, N, K))
