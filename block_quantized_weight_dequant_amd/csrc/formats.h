// The two weight block formats as the product kernels see them: byte geometry,
// the activation elements a matrix-core lane group covers, and the decode of
// that group's quant bytes into a binary16 B operand.
//
// Formats (docs.rs fuel-dispatch, "quantized (GGML) kernel contracts"):
//   Q4_0, section dequant_q4_0: 18-byte block, binary16 d (little-endian), then
//     16 bytes; the low nibble of byte j is element j, the high nibble element
//     j + 16; element = (nibble - 8) d.
//   Q8_0, section dequant_q8_0: 34-byte block, binary16 d, then 32 signed
//     bytes; element = q d.
//
// Operand geometry (v_mfma_f32_16x16x32_f16, K = 32 = one block): lane group
// g = lane / 16 supplies 8 of the block's 32 K values. Each format gives group
// g the quant bytes that are cheapest to decode together, and the activation
// side (A operand) must list the same elements in the same slot order:
//   slots 0..3 = elements lo(g) + {0, 2, 1, 3}, slots 4..7 = hi(g) + {0, 2, 1, 3}
// (the {0, 2, 1, 3} order is what a 16-bit-lane decode of a dword yields).
// Q4_0: the qs dword g, lo(g) = 4g, hi(g) = 16 + 4g. Q8_0: qs dwords 2g and
// 2g + 1, lo(g) = 8g, hi(g) = 8g + 4.
//
// Decoded values are exact binary16 integers. Q4_0 decodes the high nibbles in
// place (one shift fewer), so its slots 4..7 carry 16 (q - 8): the caller
// scales the paired activations by 2^-kHiLog2 (or the other slots by
// 2^kHiLog2 and the result back). Q8_0 needs no such factor.
#pragma once

#include "device_common.h"

namespace q4k {

// The binary16 exponent pattern of 1024.0: a half with this high byte and a
// field f < 1024 in its low bits is exactly 1024 + f.
struct FmtQ4_0 {
    static constexpr int kBytes = 18;     // bytes per 32-element block
    static constexpr int kQsDwords = 1;   // quant dwords per lane group
    static constexpr int kHiLog2 = 4;     // slots 4..7 decode to 2^kHiLog2 x the weight code
    static constexpr uint32_t kMagic = 0x64006400u;
    __host__ __device__ static constexpr int a_lo(int g) { return 4 * g; }
    __host__ __device__ static constexpr int a_hi(int g) { return 16 + 4 * g; }
    // Lane group and slot half (0: slots 0..3, 1: slots 4..7) of the run of four
    // elements that starts at element e (e % 4 == 0).
    __host__ __device__ static constexpr int a_group(int e) { return (e & 15) >> 2; }
    __host__ __device__ static constexpr int a_half(int e) { return e >> 4; }

    // qs dword x: (x & 0x000F000F) | magic is 1024 + q of bytes 0 and 2 (low
    // nibbles); (x & 0x00F000F0) | magic is 1024 + 16 q (high nibbles). With the
    // magic in a VGPR each is one v_and_or_b32.
    __device__ static __forceinline__ f16x8 decode(const uint32_t (&x)[1], uint32_t magic)
    {
        const uint32_t t = x[0] >> 8;
        const uint32_t v0 = (x[0] & 0x000F000Fu) | magic;   // elements 4g, 4g+2
        const uint32_t v1 = (t & 0x000F000Fu) | magic;      // elements 4g+1, 4g+3
        const uint32_t v2 = (x[0] & 0x00F000F0u) | magic;   // 16+4g, 16+4g+2 (x16)
        const uint32_t v3 = (t & 0x00F000F0u) | magic;      // 16+4g+1, 16+4g+3 (x16)
        const f16x2 lo_bias = {(f16)1032.0f, (f16)1032.0f};   // 1024 + 8
        const f16x2 hi_bias = {(f16)1152.0f, (f16)1152.0f};   // 1024 + 16 * 8
        const f16x2 h0 = bitcast<f16x2>(v0) - lo_bias, h1 = bitcast<f16x2>(v1) - lo_bias;
        const f16x2 h2 = bitcast<f16x2>(v2) - hi_bias, h3 = bitcast<f16x2>(v3) - hi_bias;
        return (f16x8){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    }
};

struct FmtQ8_0 {
    static constexpr int kBytes = 34;
    static constexpr int kQsDwords = 2;
    static constexpr int kHiLog2 = 0;
    static constexpr uint32_t kMagic = 0x64646464u;   // 0x64 in every byte, for v_perm_b32
    __host__ __device__ static constexpr int a_lo(int g) { return 8 * g; }
    __host__ __device__ static constexpr int a_hi(int g) { return 8 * g + 4; }
    __host__ __device__ static constexpr int a_group(int e) { return e >> 3; }
    __host__ __device__ static constexpr int a_half(int e) { return (e >> 2) & 1; }

    // qs dwords x0, x1 (bytes 8g..8g+7). Flipping bit 7 of a byte turns the
    // two's-complement q into q + 128 in 0..255; v_perm_b32 then places two such
    // bytes under the 0x64 exponent bytes of the magic, giving halves 1024 + q +
    // 128, and one packed subtraction of 1152 leaves q exactly.
    __device__ static __forceinline__ f16x8 decode(const uint32_t (&x)[2], uint32_t magic)
    {
        const uint32_t u0 = x[0] ^ 0x80808080u, u1 = x[1] ^ 0x80808080u;
        // Selector bytes (low first): 0..3 pick bytes of the second operand, 4 picks
        // byte 0 of the first (0x64).
        const uint32_t v0 = __builtin_amdgcn_perm(magic, u0, 0x04020400u);   // elements 8g, 8g+2
        const uint32_t v1 = __builtin_amdgcn_perm(magic, u0, 0x04030401u);   // 8g+1, 8g+3
        const uint32_t v2 = __builtin_amdgcn_perm(magic, u1, 0x04020400u);   // 8g+4, 8g+6
        const uint32_t v3 = __builtin_amdgcn_perm(magic, u1, 0x04030401u);   // 8g+5, 8g+7
        const f16x2 bias = {(f16)1152.0f, (f16)1152.0f};
        const f16x2 h0 = bitcast<f16x2>(v0) - bias, h1 = bitcast<f16x2>(v1) - bias;
        const f16x2 h2 = bitcast<f16x2>(v2) - bias, h3 = bitcast<f16x2>(v3) - bias;
        return (f16x8){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    }
};

// The magic of format F in a VGPR the compiler cannot fold back into a literal
// (gfx9 VOP3 instructions take no literal operand, so this keeps each decode
// step one instruction). One v_mov per kernel.
template <class F>
__device__ __forceinline__ uint32_t magic_vgpr()
{
    uint32_t m;
    if constexpr (F::kMagic == 0x64006400u)
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    else
        asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(m));
    return m;
}

// Lane group g's quant dwords of block B of a run of blocks that starts on a
// 4-byte boundary (`row`), read from LDS. The group's first quant byte is
// kBytes B + 2 + 4 kQsDwords g, which is 2 bytes past a dword boundary or on one
// depending only on B; the first case is realigned with v_alignbyte.
template <class F, int B>
__device__ __forceinline__ void read_qs(const uint32_t *row, int g, uint32_t (&x)[F::kQsDwords])
{
    constexpr int o = F::kBytes * B + 2, i0 = o / 4, sh = o % 4;
    static_assert(sh == 0 || sh == 2, "blocks start on 2-byte boundaries");
    const uint32_t *p = row + i0 + F::kQsDwords * g;
#pragma unroll
    for (int q = 0; q < F::kQsDwords; ++q) {
        if constexpr (sh != 0)
            x[q] = __builtin_amdgcn_alignbyte(p[q + 1], p[q], 2u);
        else
            x[q] = p[q];
    }
}

// The same in two steps, so that the LDS reads can be issued early and the
// realignment done later: read_qs_raw fetches the dwords that hold the group's
// bytes (one more than kQsDwords when they straddle), align_qs realigns them.
template <class F, int B>
struct QsRaw {
    static constexpr int o = F::kBytes * B + 2, i0 = o / 4, sh = o % 4;
    static constexpr int n = F::kQsDwords + (sh ? 1 : 0);
    uint32_t r[n];
};
template <class F, int B>
__device__ __forceinline__ QsRaw<F, B> read_qs_raw(const uint32_t *row, int g)
{
    QsRaw<F, B> q;
    const uint32_t *p = row + QsRaw<F, B>::i0 + F::kQsDwords * g;
#pragma unroll
    for (int i = 0; i < QsRaw<F, B>::n; ++i)
        q.r[i] = p[i];
    return q;
}
template <class F, int B>
__device__ __forceinline__ void align_qs(const QsRaw<F, B> &q, uint32_t (&x)[F::kQsDwords])
{
#pragma unroll
    for (int i = 0; i < F::kQsDwords; ++i) {
        if constexpr (QsRaw<F, B>::sh != 0)
            x[i] = __builtin_amdgcn_alignbyte(q.r[i + 1], q.r[i], 2u);
        else
            x[i] = q.r[i];
    }
}

// Dword index within such a run, and the binary16 scale bits taken from that
// dword, for block B's d.
template <class F, int B>
constexpr int d_dword() { return F::kBytes * B / 4; }
template <class F, int B>
__device__ __forceinline__ uint32_t d_from_dword(uint32_t dw)
{
    return (F::kBytes * B) % 4 ? (dw >> 16) : (dw & 0xFFFFu);
}

// The binary16 scale bits of block B of such a run.
template <class F, int B>
__device__ __forceinline__ uint32_t read_d_bits(const uint32_t *row)
{
    constexpr int o = F::kBytes * B;
    return o % 4 ? (row[o / 4] >> 16) : (row[o / 4] & 0xFFFFu);
}

// The same from global memory, for a block at any 2-byte aligned address.
template <class F>
__device__ __forceinline__ void load_qs(const uint8_t *blk, int g, uint32_t (&x)[F::kQsDwords])
{
#pragma unroll
    for (int q = 0; q < F::kQsDwords; ++q)
        x[q] = load_u32_unaligned(blk + 2 + 4 * (F::kQsDwords * g + q));
}

}  // namespace q4k
