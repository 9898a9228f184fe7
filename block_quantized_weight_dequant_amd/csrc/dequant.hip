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
// the mapping is chosen for the stores: thread f produces output float4 f, and
// a wavefront's 64 lanes store 1 KiB of consecutive bytes. Thread f reads the
// block's scale (2 bytes) and the one quant dword that holds its four values;
// the eight threads of a block share those cache lines. Each product is exact
// in f32 (at most 8 x 11 significant bits), so the output equals any correct
// evaluation bit for bit, signed zeros included.
#include "device_common.h"
#include "launch.h"

namespace q4k {

__global__ __launch_bounds__(256) void k_dequant_q4_0(const uint8_t *__restrict__ w,
                                                      float4 *__restrict__ out, size_t n_quads)
{
    size_t f = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (f >= n_quads)
        return;
    const uint8_t *blk = w + (f >> 3) * kQ4Bytes;
    unsigned part = (unsigned)f & 7;          // 0..3: low nibbles, 4..7: high nibbles
    float d = f16_bits_to_f32(load_u16(blk));
    uint32_t x = load_u32_unaligned(blk + 2 + 4 * (part & 3));
    if (part >= 4)
        x >>= 4;
    float4 v;
    v.x = (float)((int)(x & 15u) - 8) * d;
    v.y = (float)((int)((x >> 8) & 15u) - 8) * d;
    v.z = (float)((int)((x >> 16) & 15u) - 8) * d;
    v.w = (float)((int)((x >> 24) & 15u) - 8) * d;
    out[f] = v;
}

__global__ __launch_bounds__(256) void k_dequant_q8_0(const uint8_t *__restrict__ w,
                                                      float4 *__restrict__ out, size_t n_quads)
{
    size_t f = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (f >= n_quads)
        return;
    const uint8_t *blk = w + (f >> 3) * kQ8Bytes;
    unsigned part = (unsigned)f & 7;          // elements 4 part .. 4 part + 3
    float d = f16_bits_to_f32(load_u16(blk));
    const uint32_t x = load_u32_unaligned(blk + 2 + 4 * part);
    float4 v;   // each byte read as a two's-complement int8
    v.x = (float)(int8_t)(x & 0xFFu) * d;
    v.y = (float)(int8_t)((x >> 8) & 0xFFu) * d;
    v.z = (float)(int8_t)((x >> 16) & 0xFFu) * d;
    v.w = (float)(int8_t)(x >> 24) * d;
    out[f] = v;
}

hipError_t launch_dequant(WeightFormat fmt, const uint8_t *w, size_t n_blocks, float *out,
                          hipStream_t s)
{
    size_t n_quads = n_blocks * 8;
    size_t grid = (n_quads + 255) / 256;
    if (grid > 0x7fffffffu)
        return hipErrorInvalidValue;
    return launch_kernel(fmt == WeightFormat::kQ8_0 ? k_dequant_q8_0 : k_dequant_q4_0,
                         dim3((unsigned)grid), dim3(256), 0, s, w, reinterpret_cast<float4 *>(out),
                         n_quads);
}

}  // namespace q4k
