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
// Mapping: a 256-thread workgroup quantizes 32 R consecutive blocks, eight
// lanes per block, each lane holding four consecutive elements in one 16-byte
// load: lane (bl, p) of the workgroup (bl = tid / 8, p = tid % 8) takes blocks
// bl + 32 r for r < R, so a wavefront reads 1 KiB contiguously per r and has
// all R KiB in flight at once (R = 2 for large inputs, which measured faster
// than 1, 4 or 8; small ones take R = 1 so that the grid still spreads over
// the chip). The loads are unconditional
// (a block past the end re-reads the last one, whose result is dropped): a
// load under a branch would make the compiler wait for it before the join and
// serialize a lane's loads. The block maximum is reduced across the eight
// lanes with DPP moves. Every f32 operation is the single correctly rounded
// IEEE operation the rule names (HIP's default division is correctly
// rounded), so the bytes equal a sequential reference bit for bit.
//
// Output: the blocks are laid out in LDS exactly as in memory (34 or 18 bytes
// each) and written back as whole 16-byte words. A workgroup's output starts at
// a multiple of 32 R * 34 or 32 R * 18 bytes, multiples of 16, so these
// stores are aligned; only the final workgroup's last partial
// word is written byte by byte. No byte outside the output is touched, which
// the pages obtain with atomic read-modify-writes of shared words; byte stores
// make that unnecessary here. Input and output are streamed once, so loads
// and whole-word stores are non-temporal.
#include "device_common.h"
#include "launch.h"

namespace q4k {

// Blocks per eight-lane group (R) for large inputs, and the grid size below
// which a launch takes R = 1 instead.
constexpr int kQuantLaneBlocks = 2;
constexpr size_t kQuantMinGrid = 1024;

// Copy a workgroup's staged output (nbytes, a 16-byte aligned destination) to
// global memory in 16-byte words; the last partial word goes byte by byte.
__device__ __forceinline__ void store_staged(const u32x4 *stage, uint8_t *dst, unsigned nbytes,
                                             unsigned nwords)
{
    for (unsigned t = threadIdx.x; t < nwords; t += blockDim.x) {
        const unsigned off = t * 16;
        if (off + 16 <= nbytes) {
            __builtin_nontemporal_store(stage[t], reinterpret_cast<u32x4 *>(dst) + t);
        } else if (off < nbytes) {
            const uint8_t *s8 = reinterpret_cast<const uint8_t *>(stage);
            for (unsigned k = off; k < nbytes; ++k)
                dst[k] = s8[k];
        }
    }
}

// DPP lane moves within groups of eight lanes (of 32-bit values).
__device__ __forceinline__ float dpp_xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
}
__device__ __forceinline__ float dpp_xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
}
// Lane i of each eight takes lane 7 - i: after the two quad steps every lane
// holds its quad's result, so this pairs the two quads of the group.
__device__ __forceinline__ float dpp_mirror8(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
}
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_mirror8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false); }

// The lane's four elements of its block r (clamped to the workgroup's last
// block, so the load is always in bounds).
__device__ __forceinline__ f32x4 load_lane(const float *__restrict__ x, size_t b0, unsigned blk,
                                           unsigned nb_here, unsigned p)
{
    const size_t b = b0 + (blk < nb_here ? blk : nb_here - 1);
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x) + (b * 8 + p));
}

template <int R>
__global__ __launch_bounds__(256) void k_quantize_q8_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ out, size_t n_blocks)
{
    constexpr int kQuantBlocksPerWG = 32 * R;
    __shared__ u32x4 stage[kQuantBlocksPerWG * kQ8Bytes / 16];
    uint16_t *s16 = reinterpret_cast<uint16_t *>(stage);
    const unsigned tid = threadIdx.x, bl = tid >> 3, p = tid & 7;
    const size_t b0 = (size_t)blockIdx.x * kQuantBlocksPerWG;
    const size_t left = n_blocks - b0;
    const unsigned nb_here = left < (size_t)kQuantBlocksPerWG ? (unsigned)left : kQuantBlocksPerWG;

    f32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        v[r] = load_lane(x, b0, bl + 32 * r, nb_here, p);

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const unsigned blk = bl + 32 * r;
        float am = fmaxf(fmaxf(fabsf(v[r].x), fabsf(v[r].y)), fmaxf(fabsf(v[r].z), fabsf(v[r].w)));
        am = fmaxf(am, dpp_xor1(am));
        am = fmaxf(am, dpp_xor2(am));
        am = fmaxf(am, dpp_mirror8(am));

        const float d = am / 127.0f;
        int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
        if (d != 0.0f) {
            q0 = (int)roundf(v[r].x / d);
            q1 = (int)roundf(v[r].y / d);
            q2 = (int)roundf(v[r].z / d);
            q3 = (int)roundf(v[r].w / d);
        }
        const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                                ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
        if (blk < nb_here) {
            // block blk occupies bytes [34 blk, 34 blk + 34): d, then qs[0..31]
            const unsigned h = blk * (kQ8Bytes / 2);
            s16[h + 1 + 2 * p] = (uint16_t)(packed & 0xFFFFu);
            s16[h + 2 + 2 * p] = (uint16_t)(packed >> 16);
            if (p == 0)
                s16[h] = (uint16_t)f32_to_f16_bits(d);
        }
    }
    __syncthreads();
    store_staged(stage, out + b0 * kQ8Bytes, nb_here * kQ8Bytes,
                 kQuantBlocksPerWG * kQ8Bytes / 16);
}

template <int R>
__global__ __launch_bounds__(256) void k_quantize_q4_0(const float *__restrict__ x,
                                                       uint8_t *__restrict__ out, size_t n_blocks)
{
    constexpr int kQuantBlocksPerWG = 32 * R;
    __shared__ u32x4 stage[kQuantBlocksPerWG * kQ4Bytes / 16];
    uint16_t *s16 = reinterpret_cast<uint16_t *>(stage);
    const unsigned tid = threadIdx.x, bl = tid >> 3, p = tid & 7;
    const size_t b0 = (size_t)blockIdx.x * kQuantBlocksPerWG;
    const size_t left = n_blocks - b0;
    const unsigned nb_here = left < (size_t)kQuantBlocksPerWG ? (unsigned)left : kQuantBlocksPerWG;

    f32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        v[r] = load_lane(x, b0, bl + 32 * r, nb_here, p);

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const unsigned blk = bl + 32 * r;
        const float e[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        // First element of largest |x| among this lane's four (strictly larger
        // replaces), then across the block's eight lanes (larger |x| wins, the
        // lower index on a tie: an order-free rule, so any pairing of the lanes
        // gives the same winner). With no non-zero element the maximum stays +0.
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
        auto merge = [&](float oa, float ov, int oi) __attribute__((always_inline)) {
            if (oa > ba || (oa == ba && oi < bi)) {
                ba = oa;
                bv = ov;
                bi = oi;
            }
        };
        merge(dpp_xor1(ba), dpp_xor1(bv), dpp_xor1(bi));
        merge(dpp_xor2(ba), dpp_xor2(bv), dpp_xor2(bi));
        merge(dpp_mirror8(ba), dpp_mirror8(bv), dpp_mirror8(bi));
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
        // Lanes 0..3 hold elements 0..15 (low nibbles of bytes 0..15); lanes
        // 4..7 hold elements 16..31, the high nibbles of the same bytes: lane
        // p < 4 takes lane p + 4's codes (DPP row_shl:4).
        const uint32_t high = (uint32_t)__builtin_amdgcn_mov_dpp((int)codes, 0x104, 0xF, 0xF, false);
        const uint32_t bytes = codes | (high << 4);
        if (blk < nb_here) {
            const unsigned h = blk * (kQ4Bytes / 2);
            if (p < 4) {
                s16[h + 1 + 2 * p] = (uint16_t)(bytes & 0xFFFFu);
                s16[h + 2 + 2 * p] = (uint16_t)(bytes >> 16);
            }
            if (p == 0)
                s16[h] = (uint16_t)f32_to_f16_bits(d);
        }
    }
    __syncthreads();
    store_staged(stage, out + b0 * kQ4Bytes, nb_here * kQ4Bytes,
                 kQuantBlocksPerWG * kQ4Bytes / 16);
}

// R = kQuantLaneBlocks when that still gives kQuantMinGrid workgroups, else 1.
static hipError_t launch_quant(void (*k4)(const float *, uint8_t *, size_t),
                               void (*k1)(const float *, uint8_t *, size_t), const float *x,
                               size_t n_blocks, uint8_t *out, hipStream_t s)
{
    const size_t wide = 32 * (size_t)kQuantLaneBlocks;
    const bool wide_launch = (n_blocks + wide - 1) / wide >= kQuantMinGrid;
    const size_t per = wide_launch ? wide : 32;
    const size_t grid = (n_blocks + per - 1) / per;
    if (grid > 0x7fffffffu)
        return hipErrorInvalidValue;
    return launch_kernel(wide_launch ? k4 : k1, dim3((unsigned)grid), dim3(256), 0, s, x, out, n_blocks);
}

hipError_t launch_q8_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s)
{
    return launch_quant(k_quantize_q8_0<kQuantLaneBlocks>, k_quantize_q8_0<1>, x, n_blocks, out, s);
}

hipError_t launch_q4_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s)
{
    return launch_quant(k_quantize_q4_0<kQuantLaneBlocks>, k_quantize_q4_0<1>, x, n_blocks, out, s);
}

}  // namespace q4k
