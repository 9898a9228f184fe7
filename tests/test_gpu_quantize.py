"""GPU parity of q8_quantize (section quantize_q8_0 of "fuel-vulkan-kernels —
quantized (GGML) kernel contracts") and q4_quantize (GGML's Q4_0 reference
rule) against the oracle: bytes must match exactly, and no byte after the
output may change."""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import Guarded, to_dev  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

KINDS = {
    "q8": (binding.q8_quantize, oracle.q8_0_quantize, 34),
    "q4": (binding.q4_quantize, oracle.q4_0_quantize, 18),
}


def _run(kind, x: np.ndarray):
    fn, _, blk = KINDS[kind]
    xf = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = Guarded(xf.size // 32 * blk, torch.uint8)
    fn(to_dev(xf), out.view)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.host()


def _check(kind, x):
    got = _run(kind, x)
    ref = KINDS[kind][1](x)
    if not np.array_equal(got, ref):
        blk = KINDS[kind][2]
        bad = np.nonzero(got != ref)[0]
        b = bad[0] // blk
        raise AssertionError("%s: %d bytes differ; block %d got %s ref %s" % (
            kind, bad.size, b, got[b * blk:(b + 1) * blk].tobytes().hex(),
            ref[b * blk:(b + 1) * blk].tobytes().hex()))


@pytest.mark.parametrize("kind,name", [("q8", "q8_0_blocks.json"), ("q4", "q4_0_blocks.json")])
def test_hand_blocks(kind, name):
    blocks = json.load(open(os.path.join(GOLDEN, name)))["blocks"]
    x = np.array([v for b in blocks for v in b["x"]], dtype=np.float32)
    got = _run(kind, x)
    assert got.tobytes().hex(" ") == " ".join(b["bytes"] for b in blocks)


@pytest.mark.parametrize("kind", ["q8", "q4"])
@pytest.mark.parametrize("nblocks", [1, 3, 5, 31, 32, 33, 1001])
def test_ragged_tails(kind, nblocks):
    _check(kind, wl.normal_f32(2000 + nblocks, nblocks * 32, 1.0))


@pytest.mark.parametrize("kind", ["q8", "q4"])
@pytest.mark.parametrize("scale", [1e-30, 2.0 ** -10, 1e-3, 1.0, 1e4, 1e30])
def test_scales_ties_and_zero_blocks(kind, scale):
    s = np.float32(scale)
    x = wl.normal_f32(3000, (4096, 32), scale)
    x[::37] = 0.0                                  # all-zero blocks
    x[3::47, :] = np.float32(-0.0)                 # negative zeros
    # |max| tie of opposite signs: the first one in index order must win.
    x[1::41, 3] = 10 * s
    x[1::41, 7] = -10 * s
    # Rounding ties: with the block maximum chosen so that d = s, every other
    # element sits at x / d = k + 1/2 (exactly when s is a power of two).
    half = (np.arange(31, dtype=np.float32) % 16 - 8 + np.float32(0.5)) * s
    top = np.float32(127.0) * s if kind == "q8" else np.float32(-8.0) * s
    x[2::43, 0] = top
    x[2::43, 1:] = half
    _check(kind, x)


def test_q8_full_size_activation():
    spec = wl.WORKLOADS["quantize_2048x4096"]
    _check("q8", wl.activations_f32(spec["x_seed"], spec["M"], spec["K"]))


def test_q4_full_size_weight():
    spec = wl.WORKLOADS["gemm_2048x14336x4096"]
    _check("q4", wl.weights_f32(spec["w_seed"], spec["N"], spec["K"]))


@pytest.mark.parametrize("kind", ["q8", "q4"])
def test_repeat_is_bitwise_identical(kind):
    x = wl.normal_f32(4000, 32 * 777, 1.0)
    assert np.array_equal(_run(kind, x), _run(kind, x))
