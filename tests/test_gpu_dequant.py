"""GPU parity of q4_dequant and q8_dequant against the oracle: bit-exact
(sections dequant_q4_0 and dequant_q8_0 of "fuel-vulkan-kernels — quantized
(GGML) kernel contracts": every output is the exact product (nibble - 8) * d
or q * d, so a correct kernel matches bit for bit, signed zeros included)."""
import json
import os
import struct

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
from block_quantized_weight_dequant_amd import binding  # noqa: E402
from block_quantized_weight_dequant_amd import workloads as wl  # noqa: E402
from gpu_helpers import (BLOCK_BYTES, FORMATS, Guarded, f32_bits, oracle_dequant,  # noqa: E402
                         to_dev, weight_blob)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DEQUANT = {"q4_0": binding.q4_dequant, "q8_0": binding.q8_dequant}


def _run(blob: np.ndarray, fmt="q4_0"):
    nb = blob.size // BLOCK_BYTES[fmt]
    w = to_dev(blob)
    out = Guarded(nb * 32, torch.float32)
    DEQUANT[fmt](w, out.view)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.host()


def _assert_bits(got, ref):
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (f32_bits(got[~nan]) == f32_bits(ref[~nan])).all()


def test_hand_blocks():
    blocks = json.load(open(os.path.join(GOLDEN, "q4_0_blocks.json")))["blocks"]
    blob = np.frombuffer(bytes.fromhex(" ".join(b["bytes"] for b in blocks)), dtype=np.uint8)
    got = _run(blob)
    want = np.array([float(s) for b in blocks for s in b["decoded"]], dtype=np.float32)
    assert (f32_bits(got) == f32_bits(want)).all()


def test_q8_0_hand_blocks():
    # Expected values from the layout: f16 d (struct's binary16), then signed bytes.
    blocks = json.load(open(os.path.join(GOLDEN, "q8_0_blocks.json")))["blocks"]
    raw = b"".join(bytes.fromhex(b["bytes"]) for b in blocks)
    got = _run(np.frombuffer(raw, dtype=np.uint8), "q8_0")
    want = []
    for b in blocks:
        blk = bytes.fromhex(b["bytes"])
        d = struct.unpack("<e", blk[:2])[0]
        want += [np.float32(q * d) for q in struct.unpack("<32b", blk[2:])]
    assert (f32_bits(got) == f32_bits(np.array(want, dtype=np.float32))).all()


def test_every_scale_and_nibble():
    qs = bytes((j | ((15 - j) << 4)) for j in range(16))
    blob = np.frombuffer(b"".join(h.to_bytes(2, "little") + qs for h in range(65536)), np.uint8)
    _assert_bits(_run(blob), oracle.q4_0_dequant(blob))


def test_every_scale_and_code_q8_0():
    codes = np.arange(-128, 128, dtype=np.int64)
    qs = [codes[32 * i:32 * i + 32].astype(np.int8).tobytes() for i in range(8)]
    blob = np.frombuffer(b"".join(h.to_bytes(2, "little") + q for h in range(65536) for q in qs),
                         np.uint8)
    _assert_bits(_run(blob, "q8_0"), oracle.q8_0_dequant(blob))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("nb", [1, 2, 7, 8, 9, 31, 33, 1001, 65537])
def test_random_bytes_ragged(fmt, nb):
    bb = BLOCK_BYTES[fmt]
    blob = wl.uniform_bytes(1000 + nb, nb * bb)
    # keep d finite so every output is a number; NaN/inf d are covered above
    d_hi = blob[1::bb].copy()
    d_hi[(d_hi & 0x7C) == 0x7C] &= 0xBB
    blob[1::bb] = d_hi
    _assert_bits(_run(blob, fmt), oracle_dequant(fmt)(blob))


@pytest.mark.parametrize("fmt", FORMATS)
def test_ffn_weight_full_size(fmt):
    # The 14336 x 4096 FFN weight, in the launch configuration the benchmark times.
    spec = wl.WORKLOADS["dequant_14336x4096"]
    blob = weight_blob(fmt, spec["N"], spec["K"], spec["w_seed"])
    got = _run(blob, fmt)
    ref = oracle_dequant(fmt)(blob)
    assert (f32_bits(got) == f32_bits(ref)).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_repeat_is_bitwise_identical(fmt):
    blob = weight_blob(fmt, 64, 1024, 5)
    a, b = _run(blob, fmt), _run(blob, fmt)
    assert (f32_bits(a) == f32_bits(b)).all()


@pytest.mark.parametrize("fmt", FORMATS)
def test_empty_is_a_no_op(fmt):
    DEQUANT[fmt](None, None, w_bytes=0, out_elems=0)
