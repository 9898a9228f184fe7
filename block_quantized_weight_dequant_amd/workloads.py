"""Seeded synthetic inputs shaped like the benchmark workloads.

This module holds random numbers only: no step of the quantized product lives
here. The GPU path and the CPU oracle both draw their inputs from it, and
nothing else is shared between them.

Weights are f32 draws from N(0, 0.02^2) (0.02 read as the standard deviation)
that a caller turns into Q4_0 blocks with a quantizer of its own; activations
and the tensor to be Q8_0-quantized are N(0, 1) f32, and bfloat16 activations
are the high 16 bits of such f32 draws. Every draw uses numpy's
PCG64 generator (``numpy.random.default_rng(seed)``) so the bytes are the same on
every machine.
"""
from __future__ import annotations

import numpy as np

#: Named workloads: the decode GEMV (1 and 8 activation rows) against a
#: 4096 x 4096 weight, the prefill GEMM of an attention projection and of an FFN
#: up-projection, the standalone dequant of that FFN weight and the Q8_0
#: quantize of a 2048 x 4096 activation tensor. Weights are Q4_0 unless
#: ``fmt`` says Q8_0.
WORKLOADS = {
    "gemv_1x256x512": dict(kind="gemv", M=1, N=256, K=512, w_seed=100, a_seed=101),
    "gemv_1x4096x4096": dict(kind="gemv", M=1, N=4096, K=4096, w_seed=200, a_seed=201),
    "gemv_8x4096x4096": dict(kind="gemv", M=8, N=4096, K=4096, w_seed=200, a_seed=202),
    "gemm_1024x4096x4096": dict(kind="gemm", M=1024, N=4096, K=4096, w_seed=200, a_seed=203),
    "gemm_2048x14336x4096": dict(kind="gemm", M=2048, N=14336, K=4096, w_seed=400, a_seed=401),
    "dequant_14336x4096": dict(kind="dequant", N=14336, K=4096, w_seed=400),
    "quantize_2048x4096": dict(kind="quantize", M=2048, K=4096, x_seed=402),
    # The same decode, prefill and dequant shapes over Q8_0 weights (the same
    # f32 weights, quantized to Q8_0 instead).
    "q8_0_gemv_1x4096x4096": dict(kind="gemv", fmt="q8_0", M=1, N=4096, K=4096, w_seed=200,
                                  a_seed=201),
    "q8_0_gemv_8x4096x4096": dict(kind="gemv", fmt="q8_0", M=8, N=4096, K=4096, w_seed=200,
                                  a_seed=202),
    "q8_0_gemm_1024x4096x4096": dict(kind="gemm", fmt="q8_0", M=1024, N=4096, K=4096,
                                     w_seed=200, a_seed=203),
    "q8_0_gemm_2048x14336x4096": dict(kind="gemm", fmt="q8_0", M=2048, N=14336, K=4096,
                                      w_seed=400, a_seed=401),
    "q8_0_dequant_14336x4096": dict(kind="dequant", fmt="q8_0", N=14336, K=4096, w_seed=400),
    # One GPU's share when the weight rows are split eight ways: the decode GEMV
    # and the FFN prefill GEMM at N / 8.
    "gemv_1x512x4096": dict(kind="gemv", M=1, N=512, K=4096, w_seed=500, a_seed=201),
    "gemm_2048x1792x4096": dict(kind="gemm", M=2048, N=1792, K=4096, w_seed=501, a_seed=401),
    # The same share of an FFN down-projection decode (K = 14336), plain and
    # with K split across workgroups (``splitk``: the library's choice of splits).
    "gemv_1x512x14336": dict(kind="gemv", M=1, N=512, K=14336, w_seed=502, a_seed=503),
    "gemv_splitk_1x512x14336": dict(kind="gemv", splitk=True, M=1, N=512, K=14336, w_seed=502,
                                    a_seed=503),
    # Batched decode through an FFN up-projection: eight activation rows
    # against the 14336 x 4096 weight of the prefill GEMM (more row groups
    # than compute units).
    "gemv_8x14336x4096": dict(kind="gemv", M=8, N=14336, K=4096, w_seed=400, a_seed=202),
    # The decode GEMV from activations prepared once (``prepared``: the GEMV
    # alone, as when several weight matrices share one prepared input).
    "gemv_prepared_1x4096x4096": dict(kind="gemv", prepared=True, M=1, N=4096, K=4096,
                                      w_seed=200, a_seed=201),
    "gemv_prepared_8x4096x4096": dict(kind="gemv", prepared=True, M=8, N=4096, K=4096,
                                      w_seed=200, a_seed=202),
    # The decode GEMVs and prefill GEMMs with bfloat16 activations (``act="bf16"``).
    "gemv_bf16_1x4096x4096": dict(kind="gemv", act="bf16", M=1, N=4096, K=4096, w_seed=200,
                                  a_seed=201),
    "gemv_bf16_8x4096x4096": dict(kind="gemv", act="bf16", M=8, N=4096, K=4096, w_seed=200,
                                  a_seed=202),
    "q8_0_gemv_bf16_1x4096x4096": dict(kind="gemv", act="bf16", fmt="q8_0", M=1, N=4096,
                                       K=4096, w_seed=200, a_seed=201),
    "gemm_bf16_1024x4096x4096": dict(kind="gemm", act="bf16", M=1024, N=4096, K=4096, w_seed=200,
                                     a_seed=203),
    "gemm_bf16_2048x14336x4096": dict(kind="gemm", act="bf16", M=2048, N=14336, K=4096,
                                      w_seed=400, a_seed=401),
    "q8_0_gemm_bf16_2048x14336x4096": dict(kind="gemm", act="bf16", fmt="q8_0", M=2048, N=14336,
                                           K=4096, w_seed=400, a_seed=401),
    # The decode GEMVs over activations quantized to Q8_0 blocks (``act="q8_0"``:
    # the same f32 activation draws, Q8_0-quantized by the caller's quantizer).
    "gemv_q8a_1x4096x4096": dict(kind="gemv", act="q8_0", M=1, N=4096, K=4096, w_seed=200,
                                 a_seed=201),
    "gemv_q8a_8x4096x4096": dict(kind="gemv", act="q8_0", M=8, N=4096, K=4096, w_seed=200,
                                 a_seed=202),
    "q8_0_gemv_q8a_1x4096x4096": dict(kind="gemv", act="q8_0", fmt="q8_0", M=1, N=4096, K=4096,
                                      w_seed=200, a_seed=201),
    "gemm_q8a_1024x4096x4096": dict(kind="gemm", act="q8_0", M=1024, N=4096, K=4096, w_seed=200,
                                    a_seed=203),
    "gemm_q8a_2048x14336x4096": dict(kind="gemm", act="q8_0", M=2048, N=14336, K=4096,
                                     w_seed=400, a_seed=401),
}

WEIGHT_SIGMA = np.float32(0.02)


def weights_f32(seed: int, N: int, K: int) -> np.ndarray:
    """[N, K] f32 ~ N(0, 0.02^2), row-major."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, K), dtype=np.float32) * WEIGHT_SIGMA


def activations_f32(seed: int, M: int, K: int) -> np.ndarray:
    """[M, K] f32 ~ N(0, 1), row-major."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, K), dtype=np.float32)


def activations_bf16(seed: int, M: int, K: int) -> np.ndarray:
    """[M, K] bfloat16 bit patterns (uint16): the high halves of the f32 draws
    of ``activations_f32(seed, M, K)``, i.e. N(0, 1) values cut to bfloat16."""
    return (activations_f32(seed, M, K).view(np.uint32) >> 16).astype(np.uint16)


def uniform_bytes(seed: int, n: int) -> np.ndarray:
    """n uniformly random bytes (raw block streams for layout tests)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=n, dtype=np.uint8)


def uniform_ints(seed: int, low: int, high: int, shape) -> np.ndarray:
    """Integers drawn uniformly from [low, high)."""
    rng = np.random.default_rng(seed)
    return rng.integers(low, high, size=shape, dtype=np.int64)


def normal_f32(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """f32 ~ N(0, scale^2) of any shape."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
