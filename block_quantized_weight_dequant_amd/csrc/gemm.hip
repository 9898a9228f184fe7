// Prefill-shaped Q4_0 x f32 product, y[m, n] = sum_k a[m, k] * w[n, k] for any
// M, tiled through LDS onto gfx950 matrix cores.
//
// Operation: docs.rs fuel-dispatch, "quantized (GGML) kernel contracts",
// section matmul_q4_0_tiled (M > 1, 2 M N K flops, the weight streamed once
// per column block and reused across the rows of a tile), with the Q4_0 block
// of section dequant_q4_0.
//
// Design
// ------
// * A 256-thread workgroup computes a 128 x 128 tile of y; its four wavefronts
//   each own a 64 x 64 quadrant as 4 x 4 tiles of v_mfma_f32_16x16x32_f16.
//   K advances one Q4_0 block (32 elements) per step.
// * Per step the workgroup stages, in LDS, the activation slab a[128 x 32] as
//   binary16 hi = f16(a) and lo = f16((a - hi) * 2^11), and the weight slab as
//   the exact binary16 integers (q - 8) plus the same values times 2^-11, with
//   the f32 scales d of the 128 weight rows. For a in [2^e, 2^(e+1)) the
//   residual a - hi is at most 2^(e-11), so lo is at most 2^e <= |a|: no
//   overflow for |a| < 65504, and lo stays a normal binary16 unless the
//   residual is below 2^-25. The matching 2^-11 on the weights ((q - 8) 2^-11
//   is exact) makes hi * (q - 8) + lo * (q - 8) 2^-11 equal a (q - 8) to about
//   2^-22 relative (2^-36 absolute at worst), so both land in one MFMA chain.
// * Every 16 x 16 tile's block partial is scaled by its column's d into an f32
//   accumulator (d * C + acc): block partial -> scale -> sum of blocks.
// * Two LDS stages with the next step's global loads issued before the current
//   step's MFMAs; one barrier per step.
// * Tiles are renumbered so that each of the chip's 8 XCDs (which receive
//   workgroups round-robin) works on a contiguous run of tiles sharing the
//   same activation rows, which then stay in that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace q4k {

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmThreads = 256;
constexpr int kEntries = 8 * 4 * 16;   // 16-row subtiles x k-groups x rows: 512 x 16 bytes

// B operand for qs dword x (bytes 4g..4g+3 of a block): slots hold (q - 8) of
// elements 4g+0, 4g+2, 4g+1, 4g+3, 16+4g+0, 16+4g+2, 16+4g+1, 16+4g+3.
__device__ __forceinline__ f16x8 decode_plain(uint32_t x)
{
    const uint32_t v0 = (x & 0x000F000Fu) | 0x64006400u;
    const uint32_t v1 = ((x >> 8) & 0x000F000Fu) | 0x64006400u;
    const uint32_t v2 = ((x >> 4) & 0x000F000Fu) | 0x64006400u;
    const uint32_t v3 = ((x >> 12) & 0x000F000Fu) | 0x64006400u;
    const f16x2 bias = {(f16)1032.0f, (f16)1032.0f};
    f16x2 h0 = bitcast<f16x2>(v0) - bias;
    f16x2 h1 = bitcast<f16x2>(v1) - bias;
    f16x2 h2 = bitcast<f16x2>(v2) - bias;
    f16x2 h3 = bitcast<f16x2>(v3) - bias;
    return (f16x8){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

struct GemmStage {
    uint4 a[2][kEntries];   // [hi | lo][subtile][g][row] 8-half operands
    uint4 b[2][kEntries];   // [(q-8) | (q-8) 2^-11][subtile][g][col]
    float d[kGemmBN];
};

__global__ __launch_bounds__(kGemmThreads) void k_gemm_q4_0(const float *__restrict__ a,
                                                           const uint8_t *__restrict__ w,
                                                           float *__restrict__ y, int M, int N,
                                                           int K, int tiles_m, int tiles_n)
{
    __shared__ GemmStage st[2];

    // Tile order: XCD x (= workgroup id mod 8) takes tiles [x T/8, (x+1) T/8).
    const int T = tiles_m * tiles_n, L = blockIdx.x;
    const int t = (T % 8 == 0) ? (L % 8) * (T / 8) + L / 8 : L;
    const int m0 = (t / tiles_n) * kGemmBM, n0 = (t % tiles_n) * kGemmBN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * kQ4Bytes;

    // Staging role: row r of the slab, half h (elements 16h..16h+15 of the
    // activation block; qs dwords 2h, 2h+1 of the weight block).
    const int r = tid >> 1, h = tid & 1;
    const float *arow = a + (size_t)min(m0 + r, M - 1) * K + 16 * h;
    const uint8_t *wrow = w + (size_t)min(n0 + r, N - 1) * row_bytes;

    float4 av[4];
    uint32_t wx0 = 0, wx1 = 0, wdb = 0;
    auto load_step = [&](int kb) {
        const float4 *src = reinterpret_cast<const float4 *>(arow + (size_t)kb * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            av[q] = src[q];
        const uint8_t *bp = wrow + (size_t)kb * kQ4Bytes;
        wx0 = load_u32_unaligned(bp + 2 + 8 * h);
        wx1 = load_u32_unaligned(bp + 6 + 8 * h);
        wdb = load_u16(bp);
    };
    auto store_step = [&](GemmStage &s) {
        const int sub = r >> 4, i = r & 15;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const float4 v = av[gg];
            const float e[4] = {v.x, v.z, v.y, v.w};   // slot order 0, 2, 1, 3
            f16x4 hi, lo;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f16 x = (f16)e[c];
                hi[c] = x;
                lo[c] = (f16)((e[c] - (float)x) * 2048.0f);
            }
            const int idx = (sub * 4 + gg) * 16 + i;
            reinterpret_cast<uint2 *>(&s.a[0][idx])[h] = bitcast<uint2>(hi);
            reinterpret_cast<uint2 *>(&s.a[1][idx])[h] = bitcast<uint2>(lo);
        }
        const f16x8 scale = {(f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f,
                             (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f};
        const f16x8 b0 = decode_plain(wx0), b1 = decode_plain(wx1);
        const int idx0 = (sub * 4 + 2 * h) * 16 + i, idx1 = idx0 + 16;
        s.b[0][idx0] = bitcast<uint4>(b0);
        s.b[1][idx0] = bitcast<uint4>(b0 * scale);
        s.b[0][idx1] = bitcast<uint4>(b1);
        s.b[1][idx1] = bitcast<uint4>(b1 * scale);
        if (h == 0)
            s.d[r] = f16_bits_to_f32(wdb);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
            acc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};

    load_step(0);
    store_step(st[0]);
    __syncthreads();

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < nblk; ++kb) {
        GemmStage &cur = st[kb & 1];
        const bool more = kb + 1 < nblk;
        if (more)
            load_step(kb + 1);

        f16x8 ahi[4], alo[4], bq[4], bs[4];
        float dv[4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
            const int idx = ((wm * 4 + ms) * 4 + g) * 16 + li;
            ahi[ms] = bitcast<f16x8>(cur.a[0][idx]);
            alo[ms] = bitcast<f16x8>(cur.a[1][idx]);
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
            const int idx = ((wn * 4 + ns) * 4 + g) * 16 + li;
            bq[ns] = bitcast<f16x8>(cur.b[0][idx]);
            bs[ns] = bitcast<f16x8>(cur.b[1][idx]);
            dv[ns] = cur.d[(wn * 4 + ns) * 16 + li];
        }
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
                f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ms], bq[ns], zero4, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[ms], bs[ns], c, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[ms][ns][q] = fmaf(dv[ns], c[q], acc[ms][ns][q]);
            }
        }
        if (more)
            store_step(st[(kb + 1) & 1]);
        __syncthreads();
    }

    // Lane (li, g) of tile (ms, ns) holds rows 4g..4g+3 of column li.
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = m0 + wm * 64 + ms * 16 + 4 * g + q;
            if (m >= M)
                continue;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
                const int n = n0 + wn * 64 + ns * 16 + li;
                if (n < N)
                    y[(size_t)m * N + n] = acc[ms][ns][q];
            }
        }
    }
}

hipError_t launch_gemm(const float *a, const uint8_t *w, float *y, int M, int N, int K,
                       hipStream_t s)
{
    const int tiles_m = (M + kGemmBM - 1) / kGemmBM, tiles_n = (N + kGemmBN - 1) / kGemmBN;
    const long long T = (long long)tiles_m * tiles_n;
    if (T > 0x7fffffffLL)
        return hipErrorInvalidValue;
    return launch_kernel(k_gemm_q4_0, dim3((unsigned)T), dim3(kGemmThreads), 0, s, a, w, y, M, N,
                         K, tiles_m, tiles_n);
}

}  // namespace q4k
