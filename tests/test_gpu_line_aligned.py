"""The streaming GEMVs fetch whole 128-byte lines of the weight rows when every
row is a whole number of lines from a line-aligned base (K % 2048 == 0 in either
format), and the chunk's own 16-byte columns otherwise. Both load forms feed
the same arithmetic, so the same weights placed on a line boundary and 16 bytes
past one must give identical outputs, and both must meet the products' bar
against the oracle (section qmatvec_q4_0 of "fuel-vulkan-kernels — quantized
(GGML) kernel contracts"; Q8_0 blocks of section dequant_q8_0)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
import oracle  # noqa: E402
from gpu_helpers import (DEV, Guarded, assert_within_tolerance, oracle_matmul,  # noqa: E402
                         oracle_matmul_sampled, to_dev, weight_blob)

GEMV = {"q4_0": binding.q4_gemv, "q8_0": binding.q8_gemv}
GEMV_BF16 = {"q4_0": binding.q4_gemv_bf16, "q8_0": binding.q8_gemv_bf16}
PREPARE = {"q4_0": (binding.q4_gemv_prepare_bytes, binding.q4_gemv_prepare, binding.q4_gemv_prepared),
           "q8_0": (binding.q8_gemv_prepare_bytes, binding.q8_gemv_prepare, binding.q8_gemv_prepared)}
SPLITK = {"q4_0": (binding.q4_gemv_splitk_workspace_bytes, binding.q4_gemv_splitk),
          "q8_0": (binding.q8_gemv_splitk_workspace_bytes, binding.q8_gemv_splitk)}
GEMV_Q8A = {"q4_0": binding.q4_gemv_q8a, "q8_0": binding.q8_gemv_q8a}


def _placed(blob: np.ndarray, offset: int):
    """The blob on the device, starting `offset` bytes past a 128-byte line
    boundary (the backing buffer is returned too, to keep it alive)."""
    buf = torch.empty(blob.size + 256, dtype=torch.uint8, device=DEV)
    start = (-buf.data_ptr()) % 128 + offset
    view = buf[start:start + blob.size]
    view.copy_(to_dev(blob))
    assert view.data_ptr() % 128 == offset
    return buf, view


def _both(run, blob, M, N):
    """Outputs of `run(w_view, y_view)` with the weights on a line boundary and
    16 bytes past one."""
    out = []
    for off in (0, 16):
        keep, w = _placed(blob, off)
        y = Guarded(M * N, torch.float32)
        run(w, y.view)
        torch.cuda.synchronize()
        assert y.guards_intact()
        out.append(y.host().reshape(M, N))
        del keep
    return out


def _check(fmt, a_f32, blob, N, K, got, what, sampled):
    M = a_f32.shape[0]
    if sampled:
        rng = np.random.default_rng(7)
        mi = rng.integers(0, M, 2000)
        ni = rng.integers(0, N, 2000)
        mi[:2] = M - 1
        ni[:2] = (0, N - 1)
        ref, bound = oracle_matmul_sampled(fmt)(a_f32, blob, N, K, mi, ni)
        assert_within_tolerance(got[mi, ni], ref, bound, what)
    else:
        ref, bound = oracle_matmul(fmt)(a_f32, blob, N, K)
        assert_within_tolerance(got, ref, bound, what)


SHAPES = [
    (1, 4096, 4096),     # one chunk per wavefront
    (2, 4096, 4096),
    (8, 4096, 4096),
    (1, 4096, 2048),     # one 8-block chunk per wavefront
    (1, 512, 4096),      # eight weight rows per workgroup
    (1, 4100, 4096),     # row-group loops, ragged last group
    (8, 4100, 4096),
    (8, 4200, 2048),     # row-group loops over 8-block chunks
    (1, 1000, 14336),    # several chunks per wavefront
    (3, 300, 6144),
]


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_line_and_column_loads_agree(fmt, M, N, K):
    blob = weight_blob(fmt, N, K, 900 + K // 256)
    a = wl.activations_f32(901, M, K)
    a_dev = to_dev(a)
    y0, y16 = _both(lambda w, y: GEMV[fmt](a_dev, w, y, M, N, K), blob, M, N)
    np.testing.assert_array_equal(y0.view(np.uint32), y16.view(np.uint32))
    _check(fmt, a, blob, N, K, y0, "%s %dx%dx%d" % (fmt, M, N, K), sampled=N * K > 2 ** 23)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (8, 4100, 4096), (1, 1000, 14336)])
def test_line_and_column_loads_agree_bf16(fmt, M, N, K):
    blob = weight_blob(fmt, N, K, 910)
    a16 = wl.activations_bf16(911, M, K)
    a_dev = to_dev(a16.view(np.int16))
    y0, y16 = _both(lambda w, y: GEMV_BF16[fmt](a_dev, w, y, M, N, K), blob, M, N)
    np.testing.assert_array_equal(y0.view(np.uint32), y16.view(np.uint32))
    a_f32 = (a16.astype(np.uint32) << 16).view(np.float32).reshape(M, K)
    _check(fmt, a_f32, blob, N, K, y0, "bf16 %s %dx%dx%d" % (fmt, M, N, K), sampled=True)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", [(8, 4096, 4096), (4, 4100, 4096), (1, 4200, 2048), (5, 600, 14336)])
def test_line_and_column_loads_agree_prepared(fmt, M, N, K):
    nbytes, prepare, prepared = PREPARE[fmt]
    blob = weight_blob(fmt, N, K, 920)
    a = wl.activations_f32(921, M, K)
    nb = nbytes(M, K)
    prep = torch.empty(nb, dtype=torch.uint8, device=DEV)
    prepare(to_dev(a), M, K, prep)
    y0, y16 = _both(lambda w, y: prepared(prep, w, y, M, N, K), blob, M, N)
    np.testing.assert_array_equal(y0.view(np.uint32), y16.view(np.uint32))
    _check(fmt, a, blob, N, K, y0, "prepared %s %dx%dx%d" % (fmt, M, N, K), sampled=True)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_line_and_column_loads_agree_splitk(fmt):
    M, N, K = 1, 512, 14336
    ws_bytes, splitk = SPLITK[fmt]
    blob = weight_blob(fmt, N, K, 930)
    a = wl.activations_f32(931, M, K)
    a_dev = to_dev(a)
    ws = torch.empty(max(ws_bytes(M, N, K), 16), dtype=torch.uint8, device=DEV)
    y0, y16 = _both(lambda w, y: splitk(a_dev, w, y, M, N, K, workspace=ws), blob, M, N)
    np.testing.assert_array_equal(y0.view(np.uint32), y16.view(np.uint32))
    _check(fmt, a, blob, N, K, y0, "split-K %s" % fmt, sampled=False)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (8, 4096, 4096), (4, 4100, 4096), (8, 4200, 2048),
                                   (1, 1000, 14336)])
def test_line_and_column_loads_agree_q8a(fmt, M, N, K):
    """The GEMV over Q8_0-quantized activations (reading 15: the product of the
    dequantized activations) takes the same two load forms."""
    blob = weight_blob(fmt, N, K, 940)
    a_q = oracle.q8_0_quantize(wl.activations_f32(941, M, K))
    aq_dev = to_dev(a_q)
    y0, y16 = _both(lambda w, y: GEMV_Q8A[fmt](aq_dev, w, y, M, N, K), blob, M, N)
    np.testing.assert_array_equal(y0.view(np.uint32), y16.view(np.uint32))
    a_deq = oracle.q8_0_dequant(a_q).reshape(M, K)
    _check(fmt, a_deq, blob, N, K, y0, "q8a %s %dx%dx%d" % (fmt, M, N, K), sampled=True)
