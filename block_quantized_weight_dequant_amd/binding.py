"""Thin ctypes binding over libq4.so (the C ABI in include/q4.h).

Each function has the name of its C entry point and only marshals arguments:
tensors become device pointers and byte/element counts, ``stream=None`` becomes
PyTorch's current HIP stream, and a non-zero status becomes a ``Q4Error``.
Every step of the computation runs in the library's HIP kernels. There is no
fallback: if the library is missing this module raises on import.

Arguments that are pointers accept a ``torch.Tensor`` (its ``data_ptr()``), a
plain integer address, or ``None`` (NULL).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4.so")

Q4_OK = 0
Q4_ERR_NULL = 1
Q4_ERR_SHAPE = 2
Q4_ERR_SIZE = 3
Q4_ERR_ALIGN = 4
Q4_ERR_ALIAS = 5
Q4_ERR_LAUNCH = 6
Q4_ERR_WORKSPACE = 7
Q4_GEMV_MAX_ROWS = 8
Q4_GEMM_SCRATCH_BYTES = 64 << 20
SIZE_MAX = 2 ** 64 - 1

#: Every symbol include/q4.h declares.
EXPORTS = ("q4_abi_version", "q4_status_string", "q4_dequant", "q4_gemv", "q4_gemm",
           "q4_gemm_ws", "q4_gemm_workspace_bytes", "q8_dequant", "q8_gemv", "q8_gemm", "q8_gemm_ws",
           "q8_gemm_workspace_bytes", "q8_quantize", "q4_quantize", "q4_gemm_bf16",
           "q4_gemm_bf16_workspace_bytes", "q8_gemm_bf16", "q8_gemm_bf16_workspace_bytes",
           "q4_gemv_bf16", "q8_gemv_bf16", "q4_gemv_splitk", "q4_gemv_splitk_workspace_bytes",
           "q8_gemv_splitk", "q8_gemv_splitk_workspace_bytes", "q4_gemv_prepare_bytes",
           "q4_gemv_prepare", "q4_gemv_prepared", "q8_gemv_prepare_bytes", "q8_gemv_prepare",
           "q8_gemv_prepared", "q4_gemv_q8a", "q8_gemv_q8a", "q4_gemm_q8a",
           "q4_gemm_q8a_workspace_bytes", "q8_gemm_q8a", "q8_gemm_q8a_workspace_bytes")


class Q4Error(RuntimeError):
    def __init__(self, status: int, entry: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (entry, q4_status_string(status), status))


def _load_library():
    # The caller's tensors and streams belong to PyTorch's HIP runtime, and
    # PyTorch ships its own copy of it. Importing torch first makes the dynamic
    # loader resolve libq4.so's libamdhip64.so.7 to that already-loaded copy
    # (same soname); loaded the other way round, the process would hold two
    # HIP runtimes and PyTorch's stream handles would be foreign to ours.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libq4.so is not built (%s); run "
                          "`python -m block_quantized_weight_dequant_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.q4_abi_version.restype = i32
    lib.q4_abi_version.argtypes = []
    lib.q4_status_string.restype = ctypes.c_char_p
    lib.q4_status_string.argtypes = [i32]
    for f in ("q4", "q8"):
        getattr(lib, f + "_dequant").restype = i32
        getattr(lib, f + "_dequant").argtypes = [P, sz, P, sz, P]
        for g in ("_gemv", "_gemv_bf16", "_gemm"):
            getattr(lib, f + g).restype = i32
            getattr(lib, f + g).argtypes = [P, P, sz, P, i32, i32, i32, P]
        for g in ("_gemm_ws", "_gemm_bf16"):
            getattr(lib, f + g).restype = i32
            getattr(lib, f + g).argtypes = [P, P, sz, P, i32, i32, i32, P, sz, P]
        for g in ("_gemm_workspace_bytes", "_gemm_bf16_workspace_bytes"):
            getattr(lib, f + g).restype = sz
            getattr(lib, f + g).argtypes = [i32, i32, i32]
        getattr(lib, f + "_gemv_splitk").restype = i32
        getattr(lib, f + "_gemv_splitk").argtypes = [P, P, sz, P, i32, i32, i32, i32, P, sz, P]
        getattr(lib, f + "_gemv_splitk_workspace_bytes").restype = sz
        getattr(lib, f + "_gemv_splitk_workspace_bytes").argtypes = [i32, i32, i32, i32]
        getattr(lib, f + "_gemv_prepare_bytes").restype = sz
        getattr(lib, f + "_gemv_prepare_bytes").argtypes = [i32, i32]
        getattr(lib, f + "_gemv_prepare").restype = i32
        getattr(lib, f + "_gemv_prepare").argtypes = [P, i32, i32, P, sz, P]
        getattr(lib, f + "_gemv_prepared").restype = i32
        getattr(lib, f + "_gemv_prepared").argtypes = [P, sz, P, sz, P, i32, i32, i32, P]
    for name in ("q4_gemv_q8a", "q8_gemv_q8a"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, sz, P, sz, P, i32, i32, i32, P]
    for name in ("q4_gemm_q8a", "q8_gemm_q8a"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, sz, P, sz, P, i32, i32, i32, P, sz, P]
        getattr(lib, name + "_workspace_bytes").restype = sz
        getattr(lib, name + "_workspace_bytes").argtypes = [i32, i32, i32]
    for name in ("q8_quantize", "q4_quantize"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, sz, P, sz, P]
    return lib


lib = _load_library()


def _addr(x) -> int:
    """Device address of a tensor argument (an int is taken as an address).
    Host tensors are refused here: the kernels would fault on a host pointer."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("expected a device (cuda) tensor, got one on %s" % getattr(x, "device", type(x)))
    return int(x.data_ptr())


def _nbytes(x) -> int:
    return int(x.numel() * x.element_size())


def _stream(stream) -> int:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return 0
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, entry: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, entry)


def q4_abi_version() -> int:
    return int(lib.q4_abi_version())


def q4_status_string(status: int) -> str:
    return lib.q4_status_string(int(status)).decode()


def _dequant(entry, w_q, out, w_bytes, out_elems, stream) -> None:
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    oe = int(out.numel()) if out_elems is None else int(out_elems)
    _check(getattr(lib, entry)(_addr(w_q), wb, _addr(out), oe, _stream(stream)), entry)


def q4_dequant(w_q, out, w_bytes=None, out_elems=None, stream=None) -> None:
    """Q4_0 blocks (uint8 tensor) -> f32 ``out``; sizes default to the tensors'."""
    _dequant("q4_dequant", w_q, out, w_bytes, out_elems, stream)


def q8_dequant(w_q, out, w_bytes=None, out_elems=None, stream=None) -> None:
    """Q8_0 blocks (uint8 tensor) -> f32 ``out``; sizes default to the tensors'."""
    _dequant("q8_dequant", w_q, out, w_bytes, out_elems, stream)


def _gemv(entry, a, w_q, y, M, N, K, w_bytes, stream) -> None:
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    _check(getattr(lib, entry)(_addr(a), _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               _stream(stream)), entry)


def q4_gemv(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """y[M, N] = a[M, K] @ dequant(W[N, K/32])^T for 1 <= M <= 8, W Q4_0."""
    _gemv("q4_gemv", a, w_q, y, M, N, K, w_bytes, stream)


def q8_gemv(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """y[M, N] = a[M, K] @ dequant(W[N, K/32])^T for 1 <= M <= 8, W Q8_0."""
    _gemv("q8_gemv", a, w_q, y, M, N, K, w_bytes, stream)


def q4_gemv_bf16(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """As q4_gemv with ``a`` a [M, K] bfloat16 tensor (or its address)."""
    _gemv("q4_gemv_bf16", a, w_q, y, M, N, K, w_bytes, stream)


def q8_gemv_bf16(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """As q8_gemv with ``a`` a [M, K] bfloat16 tensor (or its address)."""
    _gemv("q8_gemv_bf16", a, w_q, y, M, N, K, w_bytes, stream)


def q4_gemv_prepare_bytes(M: int, K: int) -> int:
    return int(lib.q4_gemv_prepare_bytes(int(M), int(K)))


def q8_gemv_prepare_bytes(M: int, K: int) -> int:
    return int(lib.q8_gemv_prepare_bytes(int(M), int(K)))


def _gemv_prepare(entry, a, M, K, prep, prep_bytes, stream) -> None:
    pb = _nbytes(prep) if prep_bytes is None else int(prep_bytes)
    _check(getattr(lib, entry)(_addr(a), int(M), int(K), _addr(prep), pb, _stream(stream)), entry)


def q4_gemv_prepare(a, M: int, K: int, prep, prep_bytes=None, stream=None) -> None:
    """Prepared operands of the f32 activations ``a`` [M, K] for q4_gemv_prepared."""
    _gemv_prepare("q4_gemv_prepare", a, M, K, prep, prep_bytes, stream)


def q8_gemv_prepare(a, M: int, K: int, prep, prep_bytes=None, stream=None) -> None:
    """As q4_gemv_prepare, for q8_gemv_prepared."""
    _gemv_prepare("q8_gemv_prepare", a, M, K, prep, prep_bytes, stream)


def _gemv_prepared(entry, prep, w_q, y, M, N, K, prep_bytes, w_bytes, stream) -> None:
    pb = _nbytes(prep) if prep_bytes is None else int(prep_bytes)
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    _check(getattr(lib, entry)(_addr(prep), pb, _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               _stream(stream)), entry)


def q4_gemv_prepared(prep, w_q, y, M: int, N: int, K: int, prep_bytes=None, w_bytes=None,
                     stream=None) -> None:
    """y[M, N] = a @ dequant(W)^T from operands made by q4_gemv_prepare."""
    _gemv_prepared("q4_gemv_prepared", prep, w_q, y, M, N, K, prep_bytes, w_bytes, stream)


def q8_gemv_prepared(prep, w_q, y, M: int, N: int, K: int, prep_bytes=None, w_bytes=None,
                     stream=None) -> None:
    """As q4_gemv_prepared over a Q8_0 weight stream."""
    _gemv_prepared("q8_gemv_prepared", prep, w_q, y, M, N, K, prep_bytes, w_bytes, stream)


def _gemv_q8a(entry, a_q, w_q, y, M, N, K, a_bytes, w_bytes, stream) -> None:
    ab = _nbytes(a_q) if a_bytes is None else int(a_bytes)
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    _check(getattr(lib, entry)(_addr(a_q), ab, _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               _stream(stream)), entry)


def q4_gemv_q8a(a_q, w_q, y, M: int, N: int, K: int, a_bytes=None, w_bytes=None,
                stream=None) -> None:
    """y[M, N] = dequant(A_q[M, K/32]) @ dequant(W[N, K/32])^T for 1 <= M <= 8:
    activations as Q8_0 blocks (uint8 tensor, e.g. from q8_quantize), W Q4_0."""
    _gemv_q8a("q4_gemv_q8a", a_q, w_q, y, M, N, K, a_bytes, w_bytes, stream)


def q8_gemv_q8a(a_q, w_q, y, M: int, N: int, K: int, a_bytes=None, w_bytes=None,
                stream=None) -> None:
    """As q4_gemv_q8a over a Q8_0 weight stream."""
    _gemv_q8a("q8_gemv_q8a", a_q, w_q, y, M, N, K, a_bytes, w_bytes, stream)


def q4_gemm_q8a_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_gemm_q8a_workspace_bytes(int(M), int(N), int(K)))


def q8_gemm_q8a_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q8_gemm_q8a_workspace_bytes(int(M), int(N), int(K)))


def _gemm_q8a(entry, a_q, w_q, y, M, N, K, workspace, workspace_bytes, a_bytes, w_bytes,
              stream) -> None:
    ab = _nbytes(a_q) if a_bytes is None else int(a_bytes)
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    ws = workspace
    if ws is None:
        need = int(getattr(lib, entry + "_workspace_bytes")(int(M), int(N), int(K)))
        if 0 < need < SIZE_MAX:
            ws = _scratch(need, stream, y)
    if workspace_bytes is not None:
        wsb = int(workspace_bytes)
    else:
        wsb = _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0
    _check(getattr(lib, entry)(_addr(a_q), ab, _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               _addr(ws), wsb, _stream(stream)), entry)


def q4_gemm_q8a(a_q, w_q, y, M: int, N: int, K: int, workspace=None, workspace_bytes=None,
                a_bytes=None, w_bytes=None, stream=None) -> None:
    """y[M, N] = dequant(A_q[M, K/32]) @ dequant(W[N, K/32])^T for any M: activations
    as Q8_0 blocks, W Q4_0. The workspace comes from PyTorch's allocator when
    none is passed."""
    _gemm_q8a("q4_gemm_q8a", a_q, w_q, y, M, N, K, workspace, workspace_bytes, a_bytes, w_bytes,
              stream)


def q8_gemm_q8a(a_q, w_q, y, M: int, N: int, K: int, workspace=None, workspace_bytes=None,
                a_bytes=None, w_bytes=None, stream=None) -> None:
    """As q4_gemm_q8a over a Q8_0 weight stream."""
    _gemm_q8a("q8_gemm_q8a", a_q, w_q, y, M, N, K, workspace, workspace_bytes, a_bytes, w_bytes,
              stream)


def q4_gemv_splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    return int(lib.q4_gemv_splitk_workspace_bytes(int(M), int(N), int(K), int(splits)))


def q8_gemv_splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    return int(lib.q8_gemv_splitk_workspace_bytes(int(M), int(N), int(K), int(splits)))


def _gemv_splitk(entry, a, w_q, y, M, N, K, splits, w_bytes, stream, workspace,
                 workspace_bytes) -> None:
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    ws = workspace
    if ws is None:
        need = int(getattr(lib, entry + "_workspace_bytes")(int(M), int(N), int(K), int(splits)))
        if 0 < need < SIZE_MAX:
            ws = _scratch(need, stream, y)
    if workspace_bytes is not None:
        wsb = int(workspace_bytes)
    else:
        wsb = _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0
    _check(getattr(lib, entry)(_addr(a), _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               int(splits), _addr(ws), wsb, _stream(stream)), entry)


def q4_gemv_splitk(a, w_q, y, M: int, N: int, K: int, splits: int = 0, w_bytes=None,
                   stream=None, workspace=None, workspace_bytes=None) -> None:
    """As q4_gemv with K split across workgroups (``splits=0``: the library's
    choice); the partials' workspace is taken from PyTorch's caching allocator
    unless one is passed."""
    _gemv_splitk("q4_gemv_splitk", a, w_q, y, M, N, K, splits, w_bytes, stream, workspace,
                 workspace_bytes)


def q8_gemv_splitk(a, w_q, y, M: int, N: int, K: int, splits: int = 0, w_bytes=None,
                   stream=None, workspace=None, workspace_bytes=None) -> None:
    """As q4_gemv_splitk over a Q8_0 weight stream."""
    _gemv_splitk("q8_gemv_splitk", a, w_q, y, M, N, K, splits, w_bytes, stream, workspace,
                 workspace_bytes)


def q4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_gemm_workspace_bytes(int(M), int(N), int(K)))


def q8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q8_gemm_workspace_bytes(int(M), int(N), int(K)))


def _scratch(nbytes: int, stream, like):
    """A uint8 device tensor of nbytes from PyTorch's caching allocator, marked
    as in use by ``stream`` so that it is not handed out again before the work
    queued there has finished."""
    import torch
    dev = like.device if hasattr(like, "device") else torch.device("cuda", torch.cuda.current_device())
    t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if isinstance(stream, torch.cuda.Stream):
        t.record_stream(stream)
    elif isinstance(stream, int) and stream != 0:
        t.record_stream(torch.cuda.ExternalStream(stream, device=dev))
    return t


def q4_gemm_bf16_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q4_gemm_bf16_workspace_bytes(int(M), int(N), int(K)))


def q8_gemm_bf16_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib.q8_gemm_bf16_workspace_bytes(int(M), int(N), int(K)))


def _gemm(entry, a, w_q, y, M, N, K, w_bytes, stream, workspace, workspace_bytes,
          ws_entry=None) -> None:
    wb = _nbytes(w_q) if w_bytes is None else int(w_bytes)
    ws = workspace
    if ws is None:
        need = int(getattr(lib, ws_entry or entry + "_workspace_bytes")(int(M), int(N), int(K)))
        if 0 < need < SIZE_MAX:
            ws = _scratch(need, stream, y)
    if workspace_bytes is not None:
        wsb = int(workspace_bytes)
    else:
        wsb = _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0
    _check(getattr(lib, entry)(_addr(a), _addr(w_q), wb, _addr(y), int(M), int(N), int(K),
                               _addr(ws), wsb, _stream(stream)), entry)


def q4_gemm(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """y[M, N] = a[M, K] @ dequant(W[N, K/32])^T for any M, W Q4_0, with no
    workspace: the library's own device scratch (Q4_GEMM_SCRATCH_BYTES per
    GPU) serves it, so calls that overlap in time on one GPU race."""
    _gemv("q4_gemm", a, w_q, y, M, N, K, w_bytes, stream)


def q8_gemm(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None) -> None:
    """As q4_gemm, with W a Q8_0 stream (the same scratch)."""
    _gemv("q8_gemm", a, w_q, y, M, N, K, w_bytes, stream)


def q4_gemm_ws(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None, workspace=None,
               workspace_bytes=None) -> None:
    """y[M, N] = a[M, K] @ dequant(W[N, K/32])^T for any M, W Q4_0, with the
    caller's workspace.

    ``workspace=None`` takes a scratch tensor of q4_gemm_workspace_bytes(M, N, K)
    bytes from PyTorch's caching allocator for this call; pass a tensor (or an
    address with ``workspace_bytes``) to reuse one."""
    _gemm("q4_gemm_ws", a, w_q, y, M, N, K, w_bytes, stream, workspace, workspace_bytes,
          "q4_gemm_workspace_bytes")


def q8_gemm_ws(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None, workspace=None,
               workspace_bytes=None) -> None:
    """As q4_gemm_ws, with W a Q8_0 stream (workspace from q8_gemm_workspace_bytes)."""
    _gemm("q8_gemm_ws", a, w_q, y, M, N, K, w_bytes, stream, workspace, workspace_bytes,
          "q8_gemm_workspace_bytes")


def q4_gemm_bf16(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None, workspace=None,
                 workspace_bytes=None) -> None:
    """As q4_gemm_ws with ``a`` a [M, K] bfloat16 tensor (or its address); the
    workspace, from q4_gemm_bf16_workspace_bytes, is always needed."""
    _gemm("q4_gemm_bf16", a, w_q, y, M, N, K, w_bytes, stream, workspace, workspace_bytes)


def q8_gemm_bf16(a, w_q, y, M: int, N: int, K: int, w_bytes=None, stream=None, workspace=None,
                 workspace_bytes=None) -> None:
    """As q4_gemm_bf16, with W a Q8_0 stream."""
    _gemm("q8_gemm_bf16", a, w_q, y, M, N, K, w_bytes, stream, workspace, workspace_bytes)


def q8_quantize(x, out_q, n_elems=None, out_bytes=None, stream=None) -> None:
    """f32 ``x`` -> Q8_0 blocks in the uint8 tensor ``out_q``."""
    n = int(x.numel()) if n_elems is None else int(n_elems)
    ob = _nbytes(out_q) if out_bytes is None else int(out_bytes)
    _check(lib.q8_quantize(_addr(x), n, _addr(out_q), ob, _stream(stream)), "q8_quantize")


def q4_quantize(x, out_q, n_elems=None, out_bytes=None, stream=None) -> None:
    """f32 ``x`` -> Q4_0 blocks in the uint8 tensor ``out_q``."""
    n = int(x.numel()) if n_elems is None else int(n_elems)
    ob = _nbytes(out_q) if out_bytes is None else int(out_bytes)
    _check(lib.q4_quantize(_addr(x), n, _addr(out_q), ob, _stream(stream)), "q4_quantize")


def raw_status(entry: str, *args) -> int:
    """Call a C entry point with raw integer arguments and return its status
    (for tests of the argument checks)."""
    return int(getattr(lib, entry)(*args))
