// Streaming-read ceiling kernel of libq4probe.so (include/q4_probe.h): each
// thread XORs a grid-strided run of 16-byte words. Measurement only; no part
// of the Q4_0 method.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;

__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4 *__restrict__ src,
                                                         size_t n16, u32x4 *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    // Four independent loads in flight per thread per iteration.
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride],
                    x3 = src[i + 3 * stride];
        acc ^= x0 ^ x1 ^ x2 ^ x3;
    }
    for (; i < n16; i += stride)
        acc ^= src[i];
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5bd1e995u)
        *sink = acc;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int q4probe_stream_read(const void *src,
                                                                          size_t n_bytes,
                                                                          void *sink, void *stream)
{
    if (n_bytes % 16 != 0)
        return 3;
    if (n_bytes == 0)
        return 0;
    if (!src || !sink)
        return 1;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(sink)) & 15u)
        return 4;
    const size_t n16 = n_bytes / 16;
    // At least one 512-thread workgroup per CU (256), so a small buffer is
    // read by every CU at once (its fastest shape: all loads issued up
    // front); large buffers get up to 2048 workgroups of 16+ words a thread.
    size_t blocks = (n16 + 16 * kThreads - 1) / (16 * kThreads);
    if (blocks < 256)
        blocks = 256;
    if (blocks > 2048)
        blocks = 2048;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src), n16,
                       static_cast<u32x4 *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 6;
}
