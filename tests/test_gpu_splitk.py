"""GPU parity of q4_gemv_splitk / q8_gemv_splitk (the decode GEMV with K split
across workgroups; virtio-accel ADR 10, section Consequences, names the split
of the reduction over K as the way past a stalled flat GEMV geometry) against
the oracle's f64 product (sections qmatvec_q4_0, dequant_q4_0 and dequant_q8_0
of "fuel-vulkan-kernels — quantized (GGML) kernel contracts"). Every output
must satisfy |y - y_ref| <= 1e-5 * sum|a w| + 1e-6; the split partials are
added in a fixed order, so repeated calls must agree bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import (DEV, FORMATS, Guarded, assert_within_tolerance, oracle_matmul,  # noqa: E402
                         random_blocks, to_dev, weight_blob)

SPLITK = {"q4_0": binding.q4_gemv_splitk, "q8_0": binding.q8_gemv_splitk}
GEMV = {"q4_0": binding.q4_gemv, "q8_0": binding.q8_gemv}
WS = {"q4_0": binding.q4_gemv_splitk_workspace_bytes,
      "q8_0": binding.q8_gemv_splitk_workspace_bytes}


def _run(fmt, a, blob, N, K, splits, w_dev=None, workspace=None):
    M = a.shape[0]
    y = Guarded(M * N, torch.float32)
    w = to_dev(blob) if w_dev is None else w_dev
    SPLITK[fmt](to_dev(a), w, y.view, M, N, K, splits, workspace=workspace)
    torch.cuda.synchronize()
    assert y.guards_intact()
    return y.host().reshape(M, N)


def _plain(fmt, a, blob, N, K):
    M = a.shape[0]
    y = torch.empty(M * N, device=DEV)
    GEMV[fmt](to_dev(a), to_dev(blob), y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(M, N)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 512, 14336), (1, 64, 4096), (3, 300, 2048), (8, 17, 8192),
                                   (2, 129, 1024), (5, 96, 256), (1, 33, 32768)])
@pytest.mark.parametrize("splits", [0, 2, 3, 7, 64])
def test_splitk_shapes(fmt, M, N, K, splits):
    blob = weight_blob(fmt, N, K, 7 * M + N)
    a = wl.activations_f32(11 * M + K, M, K)
    got = _run(fmt, a, blob, N, K, splits)
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(got, ref, bound, "%s splitk %dx%dx%d s=%d" % (fmt, M, N, K, splits))


@pytest.mark.parametrize("fmt", FORMATS)
def test_every_code_and_random_scales(fmt):
    M, N, K = 4, 160, 4096
    blob = random_blocks(fmt, N * K // 32, 77)
    a = wl.activations_f32(78, M, K)
    got = _run(fmt, a, blob, N, K, 5)
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(got, ref, bound, "%s random blocks" % fmt)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,N,K", [(1, 64, 4096), (4, 100, 4128), (2, 50, 96)])
def test_one_split_or_general_k_is_the_plain_gemv(fmt, M, N, K):
    # One split runs the plain GEMV's kernel over the whole row; K % 256 != 0
    # takes the general kernel. Either way the result is q4_gemv's, bit for bit,
    # and no workspace is needed.
    blob = weight_blob(fmt, N, K, 3)
    a = wl.activations_f32(4, M, K)
    splits = 1 if K % 256 == 0 else 4
    assert WS[fmt](M, N, K, splits) == 0
    got = _run(fmt, a, blob, N, K, splits)
    assert np.array_equal(got.view(np.uint32), _plain(fmt, a, blob, N, K).view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
def test_agrees_with_the_plain_gemv_and_repeats_bitwise(fmt):
    M, N, K = 2, 256, 8192
    blob = weight_blob(fmt, N, K, 5)
    a = wl.activations_f32(6, M, K)
    w = to_dev(blob)
    y1 = _run(fmt, a, blob, N, K, 0, w_dev=w)
    y2 = _run(fmt, a, blob, N, K, 0, w_dev=w)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    _, bound = oracle_matmul(fmt)(a, blob, N, K)
    from oracle import tolerance
    assert (np.abs(y1.astype(np.float64) - _plain(fmt, a, blob, N, K)) <= 2 * tolerance(bound)).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_exact_workspace_with_garbage_and_guards(fmt):
    M, N, K = 3, 200, 4096
    need = WS[fmt](M, N, K, 3)
    assert need == 3 * M * N * 4
    ws = Guarded(need, torch.uint8)
    ws.view.fill_(0x7F)
    blob = weight_blob(fmt, N, K, 8)
    a = wl.activations_f32(9, M, K)
    got = _run(fmt, a, blob, N, K, 3, workspace=ws.view)
    assert ws.guards_intact()
    ref, bound = oracle_matmul(fmt)(a, blob, N, K)
    assert_within_tolerance(got, ref, bound, "exact workspace")


@pytest.mark.parametrize("fmt", FORMATS)
def test_too_small_workspace_is_rejected(fmt):
    M, N, K = 1, 64, 4096
    ws = torch.empty(WS[fmt](M, N, K, 4) - 4, dtype=torch.uint8, device=DEV)
    y = torch.full((M * N,), 3.0, device=DEV)
    with pytest.raises(binding.Q4Error) as e:
        SPLITK[fmt](to_dev(wl.activations_f32(1, M, K)), to_dev(weight_blob(fmt, N, K, 2)), y, M,
                    N, K, 4, workspace=ws)
    assert e.value.status == binding.Q4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (y == 3.0).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_graph_replays_match_eager(fmt):
    M, N, K = 1, 512, 14336
    f = SPLITK[fmt]
    blob = to_dev(weight_blob(fmt, N, K, 23))
    a = to_dev(wl.activations_f32(24, M, K))
    ws = torch.empty(WS[fmt](M, N, K, 0), dtype=torch.uint8, device=DEV)
    y_eager = torch.empty(M * N, device=DEV)
    f(a, blob, y_eager, M, N, K, 0, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty(M * N, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f(a, blob, y, M, N, K, 0, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(a, blob, y, M, N, K, 0, workspace=ws)
    for rep in range(4):
        y.fill_(float("nan"))
        f(a, blob, torch.empty_like(y), M, N, K, 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_eager.view(torch.int32)), rep


@pytest.mark.parametrize("fmt", FORMATS)
def test_empty_problems_are_no_ops(fmt):
    bb = 18 if fmt == "q4_0" else 34
    SPLITK[fmt](None, None, None, 0, 16, 256, 0, w_bytes=16 * 8 * bb)
    SPLITK[fmt](None, None, None, 3, 0, 256, 0, w_bytes=0)
