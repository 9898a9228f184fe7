"""Q4_0 block-quantized weight dequant, GEMV and GEMM on AMD MI355X (gfx950).

The compute lives in libq4.so (C ABI: include/q4.h); ``binding`` is a thin
ctypes layer over it with the same function names. ``workloads`` holds the
seeded synthetic inputs. The binding is imported on first use, so importing the
package does not require the built library.
"""
_BINDING_NAMES = ("q4_dequant", "q4_gemv", "q4_gemm", "q4_gemm_ws", "q8_quantize", "q4_quantize",
                  "q4_status_string", "q4_abi_version", "Q4Error")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
