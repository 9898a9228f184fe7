"""The GEMM entry points without a workspace argument (q4_gemm, q8_gemm), for
callers that cannot allocate: they run on the library's own device scratch.
Called through the C ABI, each must return what the workspace form
(q4_gemm_ws, q8_gemm_ws) returns for the same inputs, on two calls in a row
(the second smaller, so it runs on what the first left in the scratch), and
both must meet the products' bar against the oracle (section
matmul_q4_0_tiled of "fuel-vulkan-kernels — quantized (GGML) kernel
contracts"). At K = 4096 a chunk holds 3968 rows, so 4500 rows take two."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import (DEV, FORMATS, Guarded, assert_within_tolerance, oracle_matmul,  # noqa: E402
                         oracle_matmul_sampled, to_dev, weight_blob)

NOALLOC = {"q4_0": binding.q4_gemm, "q8_0": binding.q8_gemm}
WS = {"q4_0": binding.q4_gemm_ws, "q8_0": binding.q8_gemm_ws}


def _pair(fmt, M, N, K, seed):
    """Run both entries on the same inputs; returns (no-alloc y, workspace y,
    activations, blob) with the outputs' guard bytes checked."""
    blob = weight_blob(fmt, N, K, seed)
    a = wl.activations_f32(seed + 1, M, K)
    a_dev, w_dev = to_dev(a), to_dev(blob)
    y0 = Guarded(M * N, torch.float32)
    y1 = Guarded(M * N, torch.float32)
    NOALLOC[fmt](a_dev, w_dev, y0.view, M, N, K)
    WS[fmt](a_dev, w_dev, y1.view, M, N, K)
    torch.cuda.synchronize()
    assert y0.guards_intact() and y1.guards_intact()
    return y0.host().reshape(M, N), y1.host().reshape(M, N), a, blob


@pytest.mark.parametrize("fmt", FORMATS)
def test_no_alloc_gemm_matches_workspace_form_twice(fmt):
    # First call: two chunks of rows (3968 + 532) at K = 4096.
    M, N, K = 4500, 256, 4096
    y0, y1, a, blob = _pair(fmt, M, N, K, 71)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    mi = np.concatenate([wl.uniform_ints(73, 0, M, 3000), np.arange(3960, 3976), np.full(N, M - 1)])
    ni = np.concatenate([wl.uniform_ints(74, 0, N, 3000), np.arange(16), np.arange(N)])
    ref, bound = oracle_matmul_sampled(fmt)(a, blob, N, K, mi, ni)
    assert_within_tolerance(y0[mi, ni], ref, bound, "%s no-alloc gemm %dx%dx%d" % (fmt, M, N, K))
    # Second call, smaller: the scratch still holds the first call's data.
    M, N, K = 77, 300, 512
    y0, y1, a, blob = _pair(fmt, M, N, K, 75)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(y0, ref, bound, "%s no-alloc gemm %dx%dx%d" % (fmt, M, N, K))


@pytest.mark.parametrize("fmt", FORMATS)
def test_no_alloc_gemm_general_kernel_shapes(fmt):
    # K % 64 != 0 takes the general kernel (the row exponents alone in the
    # scratch), then a split-path call, then the general kernel again.
    for M, N, K in [(130, 96, 4128), (40, 70, 1024), (9, 33, 96)]:
        y0, y1, a, blob = _pair(fmt, M, N, K, 77 + K)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), (M, N, K)
        ref, bound = oracle_matmul(fmt)(a, blob, N, K)
        assert_within_tolerance(y0, ref, bound, "%s no-alloc gemm %dx%dx%d" % (fmt, M, N, K))


def test_no_alloc_gemm_allocates_nothing():
    # After a first call on the device (which looks up the scratch's address),
    # further calls leave the device's free memory unchanged.
    M, N, K = 300, 512, 2048
    a = to_dev(wl.activations_f32(81, M, K))
    w = to_dev(weight_blob("q4_0", N, K, 82))
    y = torch.empty(M * N, device=DEV)
    binding.q4_gemm(a, w, y, M, N, K)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        binding.q4_gemm(a, w, y, M, N, K)
        binding.q4_gemm(a, w, y, 5, N, K)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_empty_and_rejected_calls_launch_nothing():
    assert binding.raw_status("q4_gemm", None, None, 16 * 2 * 18, None, 0, 16, 64, 0) == binding.Q4_OK
    y = torch.full((64,), 3.0, device=DEV)
    st = binding.raw_status("q4_gemm", 0, 0, 18, y.data_ptr(), 1, 1, 48, 0)
    assert st == binding.Q4_ERR_SHAPE
    torch.cuda.synchronize()
    assert (y == 3.0).all()
