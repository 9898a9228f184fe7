// Block dequant on gfx950: Q4_0 or Q8_0 block stream -> dense f32.
//
// Block layouts and rules: docs.rs fuel-dispatch, "quantized (GGML) kernel
// contracts":
//   section dequant_q4_0 — 18-byte blocks (binary16 d, then 16 bytes; byte j
//     holds element j in its low nibble and element j+16 in its high nibble),
//     element = (nibble - 8) * d with d widened to f32;
//   section dequant_q8_0 — 34-byte blocks (binary16 d, then 32 signed bytes),
//     element = q * d.
//
// The operation is write-bound (18 or 34 bytes in, 128 bytes out per block), so
// the mapping is chosen for the stores: output float4 f ("quad" f) is made by
// one thread, and each store instruction of a wavefront writes 1 KiB of
// consecutive bytes. A thread makes two quads, 64 apart (a workgroup covers 512
// consecutive quads), and stores them non-temporally (global_store ... nt):
// the output is written once and consumed by later work, and streaming it
// without allocating in the caches raises the sustained write rate. Thread f
// reads the block's scale (2 bytes) and the one quant dword that holds its four
// values; the eight threads of a block share those cache lines. Each product is
// exact in f32 (at most 8 x 11 significant bits), so the output equals any
// correct evaluation bit for bit, signed zeros included.
#include "device_common.h"
#include "formats.h"
#include "launch.h"

namespace q4k {

constexpr int kDequantThreads = 256;
constexpr int kQuadsPerThread = 2;

__device__ __forceinline__ void store_nt(float4 *p, float4 v)
{
    float *o = reinterpret_cast<float *>(p);
    __builtin_nontemporal_store(v.x, o);
    __builtin_nontemporal_store(v.y, o + 1);
    __builtin_nontemporal_store(v.z, o + 2);
    __builtin_nontemporal_store(v.w, o + 3);
}

// Quad f of a Q4_0 stream: elements 4 (f % 8) .. +3 of block f / 8, which are
// low nibbles of qs dword f % 4 for parts 0..3 and high nibbles for 4..7.
__device__ __forceinline__ float4 quad_q4_0(const uint8_t *__restrict__ w, size_t f)
{
    const uint8_t *blk = w + (f >> 3) * kQ4Bytes;
    const unsigned part = (unsigned)f & 7;
    const float d = f16_bits_to_f32(load_u16(blk));
    uint32_t x = load_u32_unaligned(blk + 2 + 4 * (part & 3));
    if (part >= 4)
        x >>= 4;
    float4 v;
    v.x = (float)((int)(x & 15u) - 8) * d;
    v.y = (float)((int)((x >> 8) & 15u) - 8) * d;
    v.z = (float)((int)((x >> 16) & 15u) - 8) * d;
    v.w = (float)((int)((x >> 24) & 15u) - 8) * d;
    return v;
}

// Quad f of a Q8_0 stream: elements 4 (f % 8) .. +3 of block f / 8, the signed
// bytes of qs dword f % 8.
__device__ __forceinline__ float4 quad_q8_0(const uint8_t *__restrict__ w, size_t f)
{
    const uint8_t *blk = w + (f >> 3) * kQ8Bytes;
    const unsigned part = (unsigned)f & 7;
    const float d = f16_bits_to_f32(load_u16(blk));
    const uint32_t x = load_u32_unaligned(blk + 2 + 4 * part);
    float4 v;   // each byte read as a two's-complement int8
    v.x = (float)(int8_t)(x & 0xFFu) * d;
    v.y = (float)(int8_t)((x >> 8) & 0xFFu) * d;
    v.z = (float)(int8_t)((x >> 16) & 0xFFu) * d;
    v.w = (float)(int8_t)(x >> 24) * d;
    return v;
}

template <class F>
__global__ __launch_bounds__(kDequantThreads) void k_dequant(const uint8_t *__restrict__ w,
                                                            float4 *__restrict__ out,
                                                            size_t n_quads)
{
    const size_t base = (size_t)blockIdx.x * (kDequantThreads * kQuadsPerThread) +
                        (threadIdx.x >> 6) * (64 * kQuadsPerThread) + (threadIdx.x & 63);
#pragma unroll
    for (int r = 0; r < kQuadsPerThread; ++r) {
        const size_t f = base + 64 * r;
        if (f >= n_quads)
            return;
        if constexpr (std::is_same_v<F, FmtQ8_0>)
            store_nt(out + f, quad_q8_0(w, f));
        else
            store_nt(out + f, quad_q4_0(w, f));
    }
}

hipError_t launch_dequant(WeightFormat fmt, const uint8_t *w, size_t n_blocks, float *out,
                          hipStream_t s)
{
    const size_t n_quads = n_blocks * 8;
    const size_t per_wg = kDequantThreads * kQuadsPerThread;
    const size_t grid = (n_quads + per_wg - 1) / per_wg;
    if (grid > 0x7fffffffu)
        return hipErrorInvalidValue;
    return launch_kernel(fmt == WeightFormat::kQ8_0 ? k_dequant<FmtQ8_0> : k_dequant<FmtQ4_0>,
                         dim3((unsigned)grid), dim3(kDequantThreads), 0, s, w,
                         reinterpret_cast<float4 *>(out), n_quads);
}

}  // namespace q4k
