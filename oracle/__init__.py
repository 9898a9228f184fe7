"""Plain CPU oracle for Q4_0 / Q8_0 block quantization and the Q4_0 x f32 and
Q8_0 x f32 products.

TEST INFRASTRUCTURE, not part of the product: only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
it. It shares no code with the GPU library and never calls it; the arithmetic
lives in ``oracle.c`` (plain loops, one IEEE operation per written operation),
and this module only marshals numpy arrays into it.

What each function follows (the docs.rs page "fuel-vulkan-kernels — quantized
(GGML) kernel contracts", fuel-dispatch 0.20.71):

* ``q4_0_dequant``   section "dequant_q4_0" (block layout and (nibble - 8) * d).
* ``q8_0_quantize``  section "quantize_q8_0" (d = max|x| / 127, q = round(x / d)).
* ``q8_0_dequant``   section "dequant_q8_0" (x = qs * d).
* ``q4_0_matmul``    sections "qmatvec_q4_0" / "matmul_q4_0_tiled"
                     (y = a @ dequant(W)^T), summed in f64.
* ``q8_0_matmul``    the same product over Q8_0 weights (the quantized-matmul
                     binding picks Q4_0 or Q8_0 blocks by quant type, section
                     "qmatvec_q4_0"; weights decoded per "dequant_q8_0").
* ``q4_0_quantize``  GGML's Q4_0 reference rule as stated with the benchmark
                     workloads (not on the pages); it only makes test weights.
* ``f16_to_f32`` / ``f32_to_f16``  IEEE 754 binary16 (round to nearest even).
* ``bf16_to_f32``    bfloat16 activations widened to f32 (exact: bfloat16 is
                     the upper half of binary32); the products of bfloat16
                     activations are the f32 products of the widened values.
* ``q4_0_matmul_q8a`` / ``q8_0_matmul_q8a``  the product with activations that
                     were quantized to Q8_0 blocks along K. The geistlib issue
                     "vulkan: shader and sequencing efficiency backlog" (page 2,
                     sections Reductions and the opening summary) names an
                     activation-quantize kernel and its fusion, and defines
                     neither; read plainly, each activation row goes through
                     "quantize_q8_0" in 32-element blocks, and the product is
                     then the one of the dequantized values ("dequant_q8_0"),
                     which is exactly sum over blocks of d_w d_a sum q_w q_a.

Every function is pinned in ``tests/test_oracle_pins.py`` against values that
do not come from this module: hand-worked blocks, library routines
(``struct``'s binary16, ``numpy.float16``, ``math.fsum``), exact rational
arithmetic, brute-force searches and closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

QK = 32
Q4_0_BLOCK_BYTES = 18
Q8_0_BLOCK_BYTES = 34

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (strict IEEE flags)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
            "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sz = ctypes.c_size_t
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_bf16_to_f32_array.restype = None
    lib.orc_bf16_to_f32_array.argtypes = [P, sz, P]
    for name in ("orc_q4_0_dequant", "orc_q8_0_dequant"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [P, sz, P]
    for name in ("orc_q4_0_quantize", "orc_q8_0_quantize"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [P, sz, P]
    i32 = ctypes.c_int
    for name in ("orc_q4_0_matmul", "orc_q8_0_matmul"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, P, i32, i32, i32, P, P, i32]
    for name in ("orc_q4_0_matmul_sampled", "orc_q8_0_matmul_sampled"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, P, i32, i32, i32, P, P, ctypes.c_int64, P, P, i32]
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_max_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(arr: np.ndarray):
    return ctypes.c_void_p(arr.ctypes.data)


def _f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return x


def _u8(x) -> np.ndarray:
    return np.ascontiguousarray(np.frombuffer(bytes(x), dtype=np.uint8)
                                if isinstance(x, (bytes, bytearray)) else x, dtype=np.uint8)


# --------------------------------------------------------------------- f16

def f16_to_f32(bits: int) -> np.float32:
    return np.float32(_load().orc_f16_to_f32(int(bits)))


def f32_to_f16(value) -> int:
    return int(_load().orc_f32_to_f16(float(np.float32(value))))


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns (any shape, uint16) -> f32 values of that shape."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    if b.size:
        _load().orc_bf16_to_f32_array(_ptr(b), b.size, _ptr(out))
    return out


# -------------------------------------------------------------------- Q4_0

def q4_0_dequant(blob) -> np.ndarray:
    """Q4_0 block stream (n_blocks * 18 bytes) -> f32 [n_blocks * 32]."""
    b = _u8(blob).reshape(-1)
    if b.size % Q4_0_BLOCK_BYTES:
        raise ValueError("Q4_0 blob length %d is not a multiple of 18" % b.size)
    nb = b.size // Q4_0_BLOCK_BYTES
    out = np.empty(nb * QK, dtype=np.float32)
    if nb:
        _load().orc_q4_0_dequant(_ptr(b), nb, _ptr(out))
    return out


def q4_0_quantize(x) -> np.ndarray:
    """f32 [n] (n % 32 == 0) -> Q4_0 block stream, uint8 [n / 32 * 18]."""
    xf = _f32(x).reshape(-1)
    if xf.size % QK:
        raise ValueError("element count %d is not a multiple of 32" % xf.size)
    out = np.empty(xf.size // QK * Q4_0_BLOCK_BYTES, dtype=np.uint8)
    if xf.size:
        _load().orc_q4_0_quantize(_ptr(xf), xf.size, _ptr(out))
    return out


# -------------------------------------------------------------------- Q8_0

def q8_0_quantize(x) -> np.ndarray:
    """f32 [n] (n % 32 == 0) -> Q8_0 block stream, uint8 [n / 32 * 34]."""
    xf = _f32(x).reshape(-1)
    if xf.size % QK:
        raise ValueError("element count %d is not a multiple of 32" % xf.size)
    out = np.empty(xf.size // QK * Q8_0_BLOCK_BYTES, dtype=np.uint8)
    if xf.size:
        _load().orc_q8_0_quantize(_ptr(xf), xf.size, _ptr(out))
    return out


def q8_0_dequant(blob) -> np.ndarray:
    """Q8_0 block stream (n_blocks * 34 bytes) -> f32 [n_blocks * 32]."""
    b = _u8(blob).reshape(-1)
    if b.size % Q8_0_BLOCK_BYTES:
        raise ValueError("Q8_0 blob length %d is not a multiple of 34" % b.size)
    nb = b.size // Q8_0_BLOCK_BYTES
    out = np.empty(nb * QK, dtype=np.float32)
    if nb:
        _load().orc_q8_0_dequant(_ptr(b), nb, _ptr(out))
    return out


# ----------------------------------------------------------------- product

_BLOCK_BYTES = {"q4_0": Q4_0_BLOCK_BYTES, "q8_0": Q8_0_BLOCK_BYTES}


def _product_args(a, w_blob, N: int, K: int, fmt: str):
    af = _f32(a)
    if af.ndim == 1:
        af = af.reshape(1, -1)
    if af.shape[1] != K:
        raise ValueError("a has %d columns, K is %d" % (af.shape[1], K))
    wb = _u8(w_blob).reshape(-1)
    if K % QK or wb.size != N * (K // QK) * _BLOCK_BYTES[fmt]:
        raise ValueError("weight blob does not match N=%d K=%d" % (N, K))
    return af, wb


def _matmul(fmt, a, w_blob, N, K, threads):
    af, wb = _product_args(a, w_blob, N, K, fmt)
    M = af.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    bound = np.zeros((M, N), dtype=np.float64)
    if M and N:
        rc = getattr(_load(), "orc_%s_matmul" % fmt)(_ptr(af), _ptr(wb), M, N, K, _ptr(y),
                                                     _ptr(bound), int(threads))
        if rc:
            raise RuntimeError("oracle matmul failed (%d)" % rc)
    return y, bound


def _matmul_sampled(fmt, a, w_blob, N, K, m_idx, n_idx, threads):
    af, wb = _product_args(a, w_blob, N, K, fmt)
    M = af.shape[0]
    mi = np.ascontiguousarray(m_idx, dtype=np.int64).reshape(-1)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64).reshape(-1)
    if mi.size != ni.size:
        raise ValueError("index vectors differ in length")
    y = np.zeros(mi.size, dtype=np.float64)
    bound = np.zeros(mi.size, dtype=np.float64)
    if mi.size:
        rc = getattr(_load(), "orc_%s_matmul_sampled" % fmt)(
            _ptr(af), _ptr(wb), M, N, K, _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(bound),
            int(threads))
        if rc:
            raise RuntimeError("oracle sampled matmul failed (%d)" % rc)
    return y, bound


def q4_0_matmul(a, w_blob, N: int, K: int, threads: int = 0):
    """y[m, n] = sum_k a[m, k] * dequant(W)[n, k] in f64, and the bound
    B[m, n] = sum_k |a[m, k] * w[n, k]|. a is [M, K] f32, W is the [N, K/32]
    Q4_0 block stream. Returns (y, B), both float64 [M, N]."""
    return _matmul("q4_0", a, w_blob, N, K, threads)


def q4_0_matmul_sampled(a, w_blob, N: int, K: int, m_idx, n_idx, threads: int = 0):
    """The Q4_0 product at sampled outputs (m_idx[i], n_idx[i]); returns (y, B)
    as float64 vectors of the same length."""
    return _matmul_sampled("q4_0", a, w_blob, N, K, m_idx, n_idx, threads)


def q8_0_matmul(a, w_blob, N: int, K: int, threads: int = 0):
    """As q4_0_matmul, with W the [N, K/32] Q8_0 block stream."""
    return _matmul("q8_0", a, w_blob, N, K, threads)


def q8_0_matmul_sampled(a, w_blob, N: int, K: int, m_idx, n_idx, threads: int = 0):
    """As q4_0_matmul_sampled, with W the [N, K/32] Q8_0 block stream."""
    return _matmul_sampled("q8_0", a, w_blob, N, K, m_idx, n_idx, threads)


def _dequant_activations(a_q, M: int, K: int) -> np.ndarray:
    b = _u8(a_q).reshape(-1)
    if K % QK or b.size != M * (K // QK) * Q8_0_BLOCK_BYTES:
        raise ValueError("activation blob does not match M=%d K=%d" % (M, K))
    return q8_0_dequant(b).reshape(M, K)


def q4_0_matmul_q8a(a_q, M: int, w_blob, N: int, K: int, threads: int = 0):
    """Q8_0-quantized activations times Q4_0 weights: a_q is the [M, K/32]
    Q8_0 block stream of the activations (row m's blocks contiguous, in K
    order). The value is the f64 product of the dequantized activations
    (dequant_q8_0) with the dequantized weights, and B the matching bound, as
    q4_0_matmul. Each product of a Q8_0 value (8-bit code times an 11-bit
    scale) with a weight is exact in f64."""
    return _matmul("q4_0", _dequant_activations(a_q, M, K), w_blob, N, K, threads)


def q8_0_matmul_q8a(a_q, M: int, w_blob, N: int, K: int, threads: int = 0):
    """As q4_0_matmul_q8a, with W the [N, K/32] Q8_0 block stream."""
    return _matmul("q8_0", _dequant_activations(a_q, M, K), w_blob, N, K, threads)


def q4_0_matmul_q8a_sampled(a_q, M: int, w_blob, N: int, K: int, m_idx, n_idx, threads: int = 0):
    """q4_0_matmul_q8a at sampled outputs (m_idx[i], n_idx[i])."""
    return _matmul_sampled("q4_0", _dequant_activations(a_q, M, K), w_blob, N, K, m_idx, n_idx,
                           threads)


def q8_0_matmul_q8a_sampled(a_q, M: int, w_blob, N: int, K: int, m_idx, n_idx, threads: int = 0):
    """q8_0_matmul_q8a at sampled outputs (m_idx[i], n_idx[i])."""
    return _matmul_sampled("q8_0", _dequant_activations(a_q, M, K), w_blob, N, K, m_idx, n_idx,
                           threads)


def max_threads() -> int:
    return int(_load().orc_max_threads())


#: The products' parity bar: |y_gpu - y_ref| <= REL_TOL * B + ABS_TOL, with B
#: the bound sum_k |a[m, k] w[n, k]| that the product functions return.
REL_TOL = 1e-5
ABS_TOL = 1e-6


def tolerance(bound: np.ndarray) -> np.ndarray:
    """The product's parity tolerance, |y_gpu - y_ref| <= 1e-5 * B + 1e-6."""
    return REL_TOL * np.asarray(bound, dtype=np.float64) + ABS_TOL


def tolerance_relative(bound: np.ndarray) -> np.ndarray:
    """The bar's relative term alone, 1e-5 * B: for inputs whose results are
    so small that the absolute 1e-6 would pass any output."""
    return REL_TOL * np.asarray(bound, dtype=np.float64)
