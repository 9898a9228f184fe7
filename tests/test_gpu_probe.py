"""GPU check of the measurement-only probe library (include/q4_probe.h): the
read-and-write stream writes every output word exactly once, from the input
word its lane reads, in the proportions the quantize and dequant ceilings use."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_quantized_weight_dequant_amd import binding  # noqa: E402

LIB = os.path.join(os.path.dirname(binding.LIB_PATH), "libq4probe.so")


def _lib():
    lib = ctypes.CDLL(LIB)
    lib.q4probe_stream_rw.restype = ctypes.c_int
    lib.q4probe_stream_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("a,b", [(64, 17), (9, 64), (64, 64), (1, 64), (64, 1)])
@pytest.mark.parametrize("groups", [1, 7, 1000])
@pytest.mark.parametrize("loads,flags", [(1, 3), (2, 0), (4, 1), (8, 2)])
def test_stream_rw_writes_each_word_once(a, b, groups, loads, flags):
    lib = _lib()
    src = np.repeat(np.arange(groups * a, dtype=np.uint32), 4)         # word i = (i, i, i, i)
    s = torch.from_numpy(src.view(np.uint8)).cuda()
    guard = 64
    d = torch.full((groups * b * 16 + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    st = lib.q4probe_stream_rw(s.data_ptr(), d.data_ptr(), groups, a, b, loads, flags, sink.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    out = d.cpu().numpy()
    assert (out[groups * b * 16:] == 0xA5).all()                      # nothing past the end
    words = out[:groups * b * 16].view(np.uint32).reshape(groups * b, 4)
    want = np.empty(groups * b, np.uint32)
    hit = np.zeros(groups * b, np.int64)
    for r in range(64):
        if (r * b) & 63 < b:
            w = np.arange(groups) * b + ((r * b) >> 6)
            want[w] = np.arange(groups) * a + ((r * a) >> 6)
            hit[w] += 1
    assert (hit == 1).all()
    assert (words == want[:, None]).all()


def test_stream_rw_rejects_bad_arguments():
    lib = _lib()
    x = torch.zeros(64 * 16, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert lib.q4probe_stream_rw(x.data_ptr(), x.data_ptr(), 1, 63, 17, 1, 3, x.data_ptr(), s) == 5
    assert lib.q4probe_stream_rw(x.data_ptr(), x.data_ptr(), 1, 0, 64, 1, 3, x.data_ptr(), s) == 5
    assert lib.q4probe_stream_rw(x.data_ptr(), x.data_ptr(), 1, 64, 17, 3, 3, x.data_ptr(), s) == 5
    assert lib.q4probe_stream_rw(x.data_ptr(), x.data_ptr(), 1, 64, 17, 1, 4, x.data_ptr(), s) == 5
    assert lib.q4probe_stream_rw(None, x.data_ptr(), 1, 64, 17, 1, 3, x.data_ptr(), s) == 1
    assert lib.q4probe_stream_rw(x.data_ptr() + 4, x.data_ptr(), 1, 64, 17, 1, 3, x.data_ptr(), s) == 4
    assert lib.q4probe_stream_rw(None, None, 0, 64, 17, 1, 3, None, s) == 0
