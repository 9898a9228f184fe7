"""Helpers for the GPU parity tests: device buffers with guard regions, NaN
prefill, and the Q4_0 / Q8_0 test-weight blobs made by the oracle."""
import numpy as np
import torch

import oracle
from block_quantized_weight_dequant_amd import workloads as wl

DEV = torch.device("cuda:0")
GUARD = 256           # guard bytes on each side of an output (a multiple of 16)


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(x, copy=True, order="C")).to(DEV)


class Guarded:
    """A device output of `n` elements of `dtype` with GUARD bytes of a known
    pattern before and after it. `.view` is the (16-byte aligned) output."""

    def __init__(self, n: int, dtype: torch.dtype, fill=float("nan")):
        self.esize = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD // self.esize
        self.n = n
        self.buf = torch.empty(n + 2 * self.g, dtype=dtype, device=DEV)
        if dtype.is_floating_point:
            self.buf.fill_(fill)
            self.buf[: self.g].fill_(-1234.5)
            self.buf[self.g + n:].fill_(-1234.5)
        else:
            self.buf.fill_(0xA5 if dtype == torch.uint8 else 0x5A5A)
        self.pre = self.buf[: self.g].clone()
        self.post = self.buf[self.g + n:].clone()
        self.view = self.buf[self.g: self.g + n]
        assert self.view.data_ptr() % 16 == 0

    def guards_intact(self) -> bool:
        return bool(torch.equal(self.buf[: self.g], self.pre)
                    and torch.equal(self.buf[self.g + self.n:], self.post))

    def host(self) -> np.ndarray:
        return self.view.cpu().numpy()


def q4_blob(N: int, K: int, seed: int) -> np.ndarray:
    """Seeded N(0, 0.02^2) weights quantized to Q4_0 by the oracle."""
    return oracle.q4_0_quantize(wl.weights_f32(seed, N, K))


FORMATS = ("q4_0", "q8_0")
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34}


def weight_blob(fmt: str, N: int, K: int, seed: int) -> np.ndarray:
    """Seeded N(0, 0.02^2) weights quantized to `fmt` by the oracle."""
    return getattr(oracle, fmt + "_quantize")(wl.weights_f32(seed, N, K))


def oracle_matmul(fmt: str):
    return getattr(oracle, fmt + "_matmul")


def oracle_matmul_sampled(fmt: str):
    return getattr(oracle, fmt + "_matmul_sampled")


def oracle_dequant(fmt: str):
    return getattr(oracle, fmt + "_dequant")


def random_blocks(fmt: str, n_blocks: int, seed: int, exp_lo: int = 5, exp_hi: int = 21) -> np.ndarray:
    """Uniformly random block bytes (every code, including Q8_0's -128) with the
    scale forced finite and normal: its binary16 exponent field drawn from
    [exp_lo, exp_hi) (default 5..20, so no product overflows or is
    subnormal; 25..27 gives |d| in [1024, 8192))."""
    b = BLOCK_BYTES[fmt]
    blob = wl.uniform_bytes(seed, n_blocks * b).reshape(n_blocks, b)
    expo = wl.uniform_ints(seed + 1, exp_lo, exp_hi, n_blocks).astype(np.uint8)
    blob[:, 1] = (blob[:, 1] & 0x83) | (expo << 2)
    return blob.reshape(-1)


def assert_within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what="",
                            relative_only: bool = False):
    """|y_gpu - y_ref| <= 1e-5 * sum|a w| + 1e-6 element by element. With
    relative_only the absolute 1e-6 is dropped (1e-5 * sum|a w| alone), for
    inputs whose results are so small that the floor would pass anything."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert np.isfinite(y_gpu).all(), "%s: non-finite output" % what
    err = np.abs(y_gpu - y_ref)
    tol = oracle.tolerance_relative(bound) if relative_only else oracle.tolerance(bound)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, "%s: %d elements out of tolerance, first %s: got %r ref %r tol %r" % (
        what, len(bad), tuple(bad[0]), y_gpu[tuple(bad[0])], y_ref[tuple(bad[0])], tol[tuple(bad[0])])
    return float(np.max(err / tol)) if err.size else 0.0


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)
