// F32 -> Q8_0 and F32 -> Q4_0 block quantizers on gfx950.
//
// Q8_0 rule: docs.rs fuel-dispatch, "quantized (GGML) kernel contracts",
// section quantize_q8_0 — per 32-element block, d = max|x| / 127, the binary16
// d is stored first, then 32 signed bytes round(x / d). round() is taken half
// away from zero, x / d uses the f32 d, and an all-zero block stores d = +0 and
// q = 0.
// Q4_0 rule (not on the pages; GGML's reference quantizer): d = (element of
// largest |x|, the first on ties) / -8, q = min(15, int(x / d + 8.5)), q = 8
// when d == 0; byte j = q_j | q_{j+16} << 4 after the binary16 d.
//
// Mapping: a 256-thread workgroup quantizes 32 consecutive blocks, eight lanes
// per block, each lane holding four consecutive elements in one 16-byte load
// (a wavefront reads 1 KiB contiguously). The block maximum is reduced across
// the eight lanes with cross-lane shuffles. Every f32 operation is the single
// correctly rounded IEEE operation the rule names (HIP's default division is
// correctly rounded), so the bytes equal a sequential reference bit for bit.
//
// Output: the blocks are laid out in LDS exactly as in memory (34 or 18 bytes
// each) and written back as whole 16-byte words. A workgroup's output starts at
// a multiple of 32 * 34 = 1088 or 32 * 18 = 576 bytes, both multiples of 16, so
// these stores are aligned; only the final workgroup's last partial word is
// written byte by byte. No byte outside the output is touched, which the pages
// obtain with atomic read-modify-writes of shared words; byte stores make that
// unnecessary here.
#include "device_common.h"
#include "launch.h"

namespace q4k {

constexpr int kQuantBlocksPerWG = 32;

// Copy a workgroup's staged output (nbytes, a 16-byte aligned destination) to
// global memory in 16-byte words; the last partial word goes byte by byte.
__device__ __forceinline__ void store_staged(const uint4 *stage, uint8_t *dst, unsigned nbytes,
                                             unsigned nwords)
{
    unsigned t = threadIdx.x;
    if (t < nwords) {
        unsigned off = t * 16;
        if (off + 16 <= nbytes) {
            reinterpret_cast<uint4 *>(dst)[t] = stage[t];
        } else if (off < nbytes) {
            const uint8_t *s8 = reinterpret_cast<const uint8_t *>(stage);
            for (unsigned k = off; k < nbytes; ++k)
                dst[k] = s8[k];
        }
    }
}

__global__ __launch_bounds__(256) void k_quantize_q8_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ out, size_t n_blocks)
{
    __shared__ uint4 stage[kQuantBlocksPerWG * kQ8Bytes / 16];   // 1088 bytes
    uint16_t *s16 = reinterpret_cast<uint16_t *>(stage);
    const unsigned tid = threadIdx.x, bl = tid >> 3, p = tid & 7;
    const size_t b0 = (size_t)blockIdx.x * kQuantBlocksPerWG;
    const size_t left = n_blocks - b0;
    const unsigned nb_here = left < (size_t)kQuantBlocksPerWG ? (unsigned)left : kQuantBlocksPerWG;
    const bool valid = bl < nb_here;

    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid)
        v = reinterpret_cast<const float4 *>(x)[(b0 + bl) * 8 + p];

    float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    am = fmaxf(am, __shfl_xor(am, 1, 8));
    am = fmaxf(am, __shfl_xor(am, 2, 8));
    am = fmaxf(am, __shfl_xor(am, 4, 8));

    const float d = am / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (d != 0.0f) {
        q0 = (int)roundf(v.x / d);
        q1 = (int)roundf(v.y / d);
        q2 = (int)roundf(v.z / d);
        q3 = (int)roundf(v.w / d);
    }
    uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                      ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
    if (valid) {
        // block bl occupies bytes [34 bl, 34 bl + 34): d, then qs[0..31]
        unsigned h = bl * (kQ8Bytes / 2);
        s16[h + 1 + 2 * p] = (uint16_t)(packed & 0xFFFFu);
        s16[h + 2 + 2 * p] = (uint16_t)(packed >> 16);
        if (p == 0)
            s16[h] = (uint16_t)f32_to_f16_bits(d);
    }
    __syncthreads();
    store_staged(stage, out + b0 * kQ8Bytes, nb_here * kQ8Bytes,
                 kQuantBlocksPerWG * kQ8Bytes / 16);
}

__global__ __launch_bounds__(256) void k_quantize_q4_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ out, size_t n_blocks)
{
    __shared__ uint4 stage[kQuantBlocksPerWG * kQ4Bytes / 16];   // 576 bytes
    uint16_t *s16 = reinterpret_cast<uint16_t *>(stage);
    const unsigned tid = threadIdx.x, bl = tid >> 3, p = tid & 7;
    const size_t b0 = (size_t)blockIdx.x * kQuantBlocksPerWG;
    const size_t left = n_blocks - b0;
    const unsigned nb_here = left < (size_t)kQuantBlocksPerWG ? (unsigned)left : kQuantBlocksPerWG;
    const bool valid = bl < nb_here;

    float e[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
        float4 v = reinterpret_cast<const float4 *>(x)[(b0 + bl) * 8 + p];
        e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
    }
    // First element of largest |x| among this lane's four (strictly larger
    // replaces), then across the block's eight lanes (larger |x| wins, the lower
    // index on a tie). With no non-zero element the maximum stays +0.
    float ba = 0.0f, bv = 0.0f;
    int bi = 4 * (int)p;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (fabsf(e[c]) > ba) {
            ba = fabsf(e[c]);
            bv = e[c];
            bi = 4 * (int)p + c;
        }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        float oa = __shfl_xor(ba, m, 8);
        float ov = __shfl_xor(bv, m, 8);
        int oi = __shfl_xor(bi, m, 8);
        if (oa > ba || (oa == ba && oi < bi)) {
            ba = oa;
            bv = ov;
            bi = oi;
        }
    }
    const float d = bv / -8.0f;
    uint32_t codes = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        int q = 8;
        if (d != 0.0f) {
            float t = e[c] / d;
            t = t + 8.5f;
            q = (int)t;
            q = q > 15 ? 15 : (q < 0 ? 0 : q);
        }
        codes |= (uint32_t)q << (8 * c);
    }
    // Lanes 0..3 hold elements 0..15 (low nibbles of bytes 0..15); lanes 4..7
    // hold elements 16..31, which become the high nibbles of the same bytes.
    uint32_t high = __shfl_xor(codes, 4, 8);
    uint32_t bytes = codes | (high << 4);
    if (valid) {
        unsigned h = bl * (kQ4Bytes / 2);
        if (p < 4) {
            s16[h + 1 + 2 * p] = (uint16_t)(bytes & 0xFFFFu);
            s16[h + 2 + 2 * p] = (uint16_t)(bytes >> 16);
        }
        if (p == 0)
            s16[h] = (uint16_t)f32_to_f16_bits(d);
    }
    __syncthreads();
    store_staged(stage, out + b0 * kQ4Bytes, nb_here * kQ4Bytes,
                 kQuantBlocksPerWG * kQ4Bytes / 16);
}

static hipError_t launch_quant(void (*k)(const float *, uint8_t *, size_t), const float *x,
                               size_t n_blocks, uint8_t *out, hipStream_t s)
{
    size_t grid = (n_blocks + kQuantBlocksPerWG - 1) / kQuantBlocksPerWG;
    if (grid > 0x7fffffffu)
        return hipErrorInvalidValue;
    return launch_kernel(k, dim3((unsigned)grid), dim3(256), 0, s, x, out, n_blocks);
}

hipError_t launch_q8_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s)
{
    return launch_quant(k_quantize_q8_0, x, n_blocks, out, s);
}

hipError_t launch_q4_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s)
{
    return launch_quant(k_quantize_q4_0, x, n_blocks, out, s);
}

}  // namespace q4k
