// Prefill-shaped block-quantized x f32 product, y[m, n] = sum_k a[m, k] w[n, k]
// for any M, tiled through LDS onto gfx950 matrix cores, for Q4_0 and Q8_0
// weight streams.
//
// Operation: docs.rs fuel-dispatch, "quantized (GGML) kernel contracts",
// section matmul_q4_0_tiled (M > 1, 2 M N K flops, the weight streamed once
// per column block and reused across the rows of a tile), with the blocks of
// sections dequant_q4_0 and dequant_q8_0 (the quantized-matmul binding picks
// either by quant type).
//
// Range: every activation row m is first scaled by a power of two 2^p_m
// (k_row_exp_f32) that puts its largest magnitude in [2^14, 2^15), so any
// finite f32 row fits the binary16 terms below; each result row is scaled back
// by 2^-p_m (exact unless it lands among the f32 subnormals).
//
// Summation order (worst case, u = 2^-24): the two-term split is within 2^-22
// (4u) of each scaled activation; an MFMA block partial adds the lo products
// (each at most 2^-11 of its hi product) first and the hi products onto them,
// about 32u; the scale FMAs d * C + acc then add at most kMaxChain block
// partials in sequence per accumulator, the K groups' tiles are added once,
// and longer K is cut into segments (separate launches, each adding its part
// into y). With S segments the error is at most (36 + kMaxChain + S) u of
// sum |a w|: 150u < 1e-5 for K up to 14336, and below 1e-5 while S <= 19.
//
// General kernel (k_gemm_any, any K % 32 == 0)
// -------------------------------------------
// * A 256-thread workgroup computes a 128 x 128 tile of y; its four wavefronts
//   each own a 64 x 64 quadrant as 4 x 4 tiles of v_mfma_f32_16x16x32_f16.
//   K advances one block (32 elements) per step.
// * Per step the workgroup stages, in LDS, the activation slab a[128 x 32] as
//   binary16 hi = f16(a) and lo = f16((a - hi) * 2^11), and the weight slab as
//   the exact binary16 weight codes plus the same values times 2^-11, with
//   the f32 scales d of the 128 weight rows. For a in [2^e, 2^(e+1)) the
//   residual a - hi is at most 2^(e-11), so lo is at most 2^e <= |a|: no
//   overflow once the row is scaled below 2^15, and lo stays a normal binary16
//   unless the residual is below 2^-25. The matching 2^-11 on the weights
//   (exact) makes hi * c + lo * c 2^-11 equal a c to about 2^-22 relative, so
//   both land in one MFMA chain.
// * Every 16 x 16 tile's block partial is scaled by its column's d into an f32
//   accumulator (d * C + acc): block partial -> scale -> sum of blocks.
// * Two LDS stages with the next step's global loads issued before the current
//   step's MFMAs; one barrier per step.
// * Tiles are renumbered so that each of the chip's 8 XCDs (which receive
//   workgroups round-robin) works on a contiguous run of tiles sharing the
//   same activation rows, which then stay in that XCD's L2.
// The slot order of the operands and the decode of the weight bytes are the
// format's (formats.h); where the decode leaves a factor 2^kHiLog2 on slots
// 4..7 (Q4_0), the activations of those slots carry 2^-kHiLog2.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "formats.h"
#include "launch.h"
#include "validate.h"

namespace q4k {

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmThreads = 256;
constexpr int kEntries = 8 * 4 * 16;   // 16-row subtiles x k-groups x rows: 512 x 16 bytes

struct GemmStage {
    uint4 a[2][kEntries];   // [hi | lo][subtile][g][row] 8-half operands
    uint4 b[2][kEntries];   // [code | code 2^-11][subtile][g][col]
    float d[kGemmBN];
};

// One K segment of the product: a and w point at block kb0 of row 0 (a row
// of a is K floats, a row of w K/32 blocks), and the segment spans nblk
// blocks. row_exp: when not null, row m of the result is scaled back by
// 2^-row_exp[m]; scale_in says whether the kernel scales row m of a by
// 2^row_exp[m] itself (the f32 path) or a was scaled beforehand (the bfloat16
// and Q8_0-activation paths). accumulate: add the segment's result to y.
template <class F>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_any(const float *__restrict__ a,
                                                          const uint8_t *__restrict__ w,
                                                          float *__restrict__ y, int M, int N,
                                                          int K, int nblk, int tiles_m, int tiles_n,
                                                          const int *__restrict__ row_exp,
                                                          int scale_in, int accumulate)
{
    __shared__ GemmStage st[2];

    // Tile order: XCD x (= workgroup id mod 8) takes tiles [x T/8, (x+1) T/8).
    const int T = tiles_m * tiles_n, L = blockIdx.x;
    const int t = (T % 8 == 0) ? (L % 8) * (T / 8) + L / 8 : L;
    const int m0 = (t / tiles_n) * kGemmBM, n0 = (t % tiles_n) * kGemmBN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t row_bytes = (size_t)(K >> 5) * F::kBytes;

    // Staging role: row r of the slab, half h (elements 16h..16h+15 of the
    // activation block; the quant bytes of lane groups 2h and 2h+1 of the
    // weight block).
    const int r = tid >> 1, h = tid & 1;
    const int ar = min(m0 + r, M - 1);
    const float *arow = a + (size_t)ar * K + 16 * h;
    const uint8_t *wrow = w + (size_t)min(n0 + r, N - 1) * row_bytes;
    const int pin = scale_in ? row_exp[ar] : 0;

    float4 av[4];
    uint32_t wx[2][F::kQsDwords];
    uint32_t wdb = 0;
    auto load_step = [&](int kb) {
        const float4 *src = reinterpret_cast<const float4 *>(arow + (size_t)kb * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            av[q] = src[q];
        const uint8_t *bp = wrow + (size_t)kb * F::kBytes;
        load_qs<F>(bp, 2 * h, wx[0]);
        load_qs<F>(bp, 2 * h + 1, wx[1]);
        wdb = load_u16(bp);
    };
    auto store_step = [&](GemmStage &s) {
        const int sub = r >> 4, i = r & 15;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // Elements 16h + 4q .. + 3 fill one slot half of one lane group.
            // Slots 4..7 meet weights decoded at 2^kHiLog2 x their code: they
            // carry a further 2^-kHiLog2 (exact).
            const int e0 = 16 * h + 4 * q, gg = F::a_group(e0), half = F::a_half(e0);
            const int sh = pin - (half ? F::kHiLog2 : 0);
            const float4 v = av[q];
            const float e[4] = {ldexpf(v.x, sh), ldexpf(v.z, sh), ldexpf(v.y, sh),
                                ldexpf(v.w, sh)};   // slot order 0, 2, 1, 3
            f16x4 hi, lo;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f16 x = (f16)e[c];
                hi[c] = x;
                lo[c] = (f16)((e[c] - (float)x) * 2048.0f);
            }
            const int idx = (sub * 4 + gg) * 16 + i;
            reinterpret_cast<uint2 *>(&s.a[0][idx])[half] = bitcast<uint2>(hi);
            reinterpret_cast<uint2 *>(&s.a[1][idx])[half] = bitcast<uint2>(lo);
        }
        const f16x8 scale = {(f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f,
                             (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f, (f16)0x1p-11f};
        const f16x8 b0 = F::decode(wx[0], F::kMagic), b1 = F::decode(wx[1], F::kMagic);
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
                // The small lo products first, the hi products onto them.
                f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[ms], bs[ns], zero4, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[ms], bq[ns], c, 0, 0, 0);
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
            const int pe = row_exp ? row_exp[m] : 0;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns) {
                const int n = n0 + wn * 64 + ns * 16 + li;
                if (n < N) {
                    float v = ldexpf(acc[ms][ns][q], -pe);
                    if (accumulate)
                        v += y[(size_t)m * N + n];
                    y[(size_t)m * N + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-activation path, for K % 64 == 0 (K splits into pairs of blocks, and a
// weight row, a whole number of pairs of 36 or 68 bytes, starts on a 4-byte
// boundary).
//
// * k_gemm_prep_f32 finds the row exponents and writes the activations once,
//   already split (hi = f16(a), lo = f16((a - hi) 2^11), after the row's power
//   of two) and laid out as the matrix cores' A operands:
//   16-byte operand [mt][kb][hl][sub][lane] holds, for row 128 mt + 16 sub +
//   lane % 16 and block kb, the slots of lane group g = lane / 16 in the
//   format's order (formats.h), hi for hl = 0 and lo for hl = 1. Rows past M
//   are zero. The split then costs one pass over the activations instead of
//   one per column tile, and a workgroup's activation slab for a pair of
//   blocks is 32 contiguous KB.
// * k_gemm_split: a 512-thread workgroup computes a 128 x 128 tile. Its eight
//   wavefronts are two K groups of four: group kg takes the even (kg = 0) or
//   odd (kg = 1) block of each pair, and wavefront (wm, wn) of a group owns a
//   64 x 64 quadrant as 4 x 4 MFMA tiles. Two wavefronts per SIMD hide each
//   other's VALU work and latencies; the two groups' partial tiles are added
//   once, through LDS, at the end.
// * Per pair of blocks the workgroup stages the 32 KB activation slab and the
//   raw weight bytes of the pair (36 or 68 per row) of its 128 rows in LDS,
//   with direct-to-LDS loads in a ring (below). Each wavefront decodes its own
//   B operands from the raw bytes: the quant bytes of lane group g for column
//   lane % 16, realigned with v_alignbyte where they straddle dwords, become
//   the binary16 codes and the same times 2^-11, and d stays binary16 until
//   the scale FMA.
// * Accumulation as in the general kernel: two chained MFMAs per 16 x 16 tile
//   and block (lo x code 2^-11, then hi x code onto it), then d * C + acc in
//   f32.

constexpr int kOpsPerBlockTile = 2 * 8 * 64;   // 16-byte A operands per (128-row tile, block)

// The one-launch preparations (k_gemm_prep_f32, k_gemm_prep_bf16,
// k_gemm_prep_q8a): one wavefront per row of a 16-row group.
constexpr int kPrepWaves = 16;
constexpr long long kPrepTarget = 256;   // workgroups the preparation aims for

// Blocks per K part of a fused preparation: enough parts for about
// kPrepTarget workgroups over `groups` row groups, each part a whole number
// of `unit` blocks and at least one unit per wavefront.
static int prep_part_blocks(long long groups, int nblk, int unit)
{
    const long long units = nblk / unit;
    const long long parts = max(1LL, min(units / kPrepWaves, (kPrepTarget + groups - 1) / groups));
    return (int)((units + parts - 1) / parts) * unit;
}

// Order a wavefront's LDS writes before its later LDS reads (its LDS
// operations execute in issue order; the fences keep the compiler's order).
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Largest of a non-negative 32-bit value over the wavefront, in every lane:
// DPP within quads, half-rows and rows, then one readlane per row.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    int x = (int)v;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));   // row_half_mirror
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));   // row_mirror
    return max(max((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
               max((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

// The split of one (16-row group R, block kb) by one wavefront: lane l loads
// 16-byte piece l % 8 of rows l / 8 and 8 + l / 8 (whole 128-byte block rows,
// eight lanes per row; rows past M re-read row M - 1 and are written as
// zeros), and a padded LDS tile ([16 rows][9 pieces]: conflict-free both
// ways) hands lane (g, li) its two pieces, the slots of lane group g of row
// li, which it splits with row li's power of two p.
struct SplitRows {
    float4 v[2];
};

__device__ __forceinline__ SplitRows split_load(const float *__restrict__ a, int M, int K,
                                                long long R, int kb, int lane)
{
    const int pr = lane >> 3, pc = lane & 7;
    SplitRows x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const long long row = min(R * 16 + pr + 8 * i, (long long)M - 1);
        x.v[i] = *reinterpret_cast<const float4 *>(a + row * K + (long long)kb * 32 + 4 * pc);
    }
    return x;
}

template <class F>
__device__ __forceinline__ void split_store(const SplitRows &x, int p, u32x4 *__restrict__ ahl,
                                            int M, int nblk, long long R, int kb, float4 *tile,
                                            int lane)
{
    const int pr = lane >> 3, pc = lane & 7;
    wave_lds_fence();   // the tile's previous reads precede these writes
#pragma unroll
    for (int i = 0; i < 2; ++i)
        tile[(pr + 8 * i) * 9 + pc] = x.v[i];
    wave_lds_fence();
    const int li = lane & 15, g = lane >> 4;
    const long long m = R * 16 + li;
    f16x8 hi = {}, lo = {};
    if (m < M) {
        const float4 L = tile[li * 9 + F::a_lo(g) / 4];
        const float4 H = tile[li * 9 + F::a_hi(g) / 4];
        // Slots 4..7 meet weights decoded at 2^kHiLog2 x their code: they carry
        // a further 2^-kHiLog2 (exact), so every product is a 2^p times the code.
        const int ph = p - F::kHiLog2;
        const float e[8] = {ldexpf(L.x, p),  ldexpf(L.z, p),  ldexpf(L.y, p),  ldexpf(L.w, p),
                            ldexpf(H.x, ph), ldexpf(H.z, ph), ldexpf(H.y, ph), ldexpf(H.w, ph)};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const f16 h = (f16)e[s];
            hi[s] = h;
            lo[s] = (f16)((e[s] - (float)h) * 2048.0f);
        }
    }
    const long long mt = R >> 3;
    const long long idx = (mt * nblk + kb) * kOpsPerBlockTile + (R & 7) * 64 + lane;
    ahl[idx] = bitcast<u32x4>(hi);
    ahl[idx + 8 * 64] = bitcast<u32x4>(lo);
}

constexpr int kSplitGemmThreads = 512;
// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9: 32-bit data format.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kLdsBytes = 160 * 1024;   // LDS of one gfx950 compute unit

// Per-format geometry of one pair of blocks.
template <class F>
struct PairGeom {
    static constexpr int kDwords = 2 * F::kBytes / 4;                 // raw dwords per row: 9 or 17
    static constexpr int kBDwords = kGemmBN * kDwords;                // ... per tile
    // A weight stage holds two consecutive pairs: row r's 2 kDwords dwords
    // (pair 2Q, then pair 2Q + 1, contiguous in the row) at r * 2 kDwords.
    static constexpr int kBQDwords = 2 * kBDwords;                    // ... per stage
    static constexpr int kBQLoads = (kBQDwords + 255) / 256;          // 4-byte loads per 256 threads
    static constexpr int kBQSlots = kBQLoads * 256;                   // LDS dwords per stage
};

// Ring depths: a pair's activation slab is loaded kA steps before the pair is
// computed; the raw weight bytes go two pairs per stage into kBQ stages, each
// loaded 2 kBQ - 1 steps before its first pair. Measured on MI355X
// (2048 x 14336 x 4096, one process), with one pair per weight stage: Q4_0
// is fastest at 4 activation stages (3 costs 2.5 %), Q8_0, whose four
// activation stages do not fit next to its weight stages, at 3; two pairs
// per weight stage gained about 1 %, and a third weight stage (five steps
// ahead) cost 1-3 % on every form.
// HO ("hi only") selects the bfloat16-activation form: one binary16 term per
// activation (exact, see k_gemm_prep_bf16), so a slab is half the size and a
// tile-block needs one MFMA instead of two. With its 128 x 32 wavefront tiles
// both formats are fastest at 4 activation stages (5 costs 3-4 %; 3 stages of
// its slab would not hold the final reduction).
template <class F, bool HO>
struct RingDepth;
template <>
struct RingDepth<FmtQ4_0, false> {
    static constexpr int kA = 4, kBQ = 2;
};
template <>
struct RingDepth<FmtQ8_0, false> {
    static constexpr int kA = 3, kBQ = 2;
};
template <>
struct RingDepth<FmtQ4_0, true> {
    static constexpr int kA = 4, kBQ = 2;
};
template <>
struct RingDepth<FmtQ8_0, true> {
    static constexpr int kA = 4, kBQ = 2;
};

// 16-byte A operands per (128-row tile, block): hi and lo, or hi only.
template <bool HO>
constexpr int slab_ops() { return HO ? kOpsPerBlockTile / 2 : kOpsPerBlockTile; }

template <class F, bool HO>
struct SplitLds {
    static constexpr int DA = RingDepth<F, HO>::kA, DBQ = RingDepth<F, HO>::kBQ;
    u32x4 a[DA][2 * slab_ops<HO>()];          // a pair's slab: [kg][hl][sub][lane], as in the workspace
    uint32_t b[DBQ][PairGeom<F>::kBQSlots];   // two pairs: [row][2 kDwords]; slots past the tile are never read
};
static_assert(sizeof(SplitLds<FmtQ4_0, false>) <= kLdsBytes &&
                  sizeof(SplitLds<FmtQ8_0, false>) <= kLdsBytes &&
                  sizeof(SplitLds<FmtQ4_0, true>) <= kLdsBytes &&
                  sizeof(SplitLds<FmtQ8_0, true>) <= kLdsBytes,
              "the rings fit in LDS");

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) lgkmcnt(0), expcnt unchanged.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

// Wait until this wavefront has at most `vm` vector-memory operations
// outstanding and all its LDS operations are done, then meet the workgroup.
// A raw s_barrier: __syncthreads() would also wait for every outstanding
// direct-to-LDS load, which are meant to stay in flight. The empty asm
// statements keep the compiler from moving LDS accesses across it.
template <int VM>
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Loads a loading wavefront may still have in flight at the barrier that ends
// step p (parity par) of k_gemm_split's ring, when pair p + 2 must be
// complete: step s issues na A loads (pair s + da) and, for odd s, then nb B
// loads (pairs s + lb and s + lb + 1), in that order; a load is identified by
// (step, slot), and the count is the loads after the last one pair p + 2 needs.
constexpr int ring_in_flight(int par, int da, int lb, int na, int nb)
{
    const int p = 1000 + par, q = p + 2;
    const int a_step = q - da, a_slot = na - 1;
    const int b_step = 2 * (q / 2) - lb, b_slot = na + nb - 1;
    int ls = a_step, lk = a_slot;
    if (b_step > ls || (b_step == ls && b_slot > lk))
        ls = b_step, lk = b_slot;
    int n = 0;
    for (int st = ls; st <= p; ++st) {
        const int slots = na + ((st & 1) ? nb : 0);
        for (int k = 0; k < slots; ++k)
            if (st > ls || k > lk)
                ++n;
    }
    return n;
}

// One K segment of the product: ahl points at the operands of block kb0 of
// the first row tile (a row tile holds nblk_row blocks of operands) and w at
// block kb0 of weight row 0 (a weight row is nblk_row blocks); the segment
// spans nblk blocks (even). row_exp: per-row exponents of the activation
// operands, undone on the result rows (always for the bfloat16 form, HO; for
// the two-term form when not null). accumulate: add the segment's result to y.
template <class F, bool HO>
__global__ __launch_bounds__(kSplitGemmThreads) void k_gemm_split(
    const u32x4 *__restrict__ ahl, const uint8_t *__restrict__ w, float *__restrict__ y, int M,
    int N, int nblk_row, int nblk, int tiles_m, int tiles_n, const int *__restrict__ row_exp,
    int accumulate)
{
    using G = PairGeom<F>;
    // MFMA tiles per wavefront: the hi-only form takes 128 rows x 32 columns
    // (8 x 2), so no two wavefronts of a K group decode the same weight
    // columns; the two-term form keeps 64 x 64 (4 x 4), which leaves room for
    // its lo operands in registers.
    constexpr int RM = HO ? 8 : 4, CN = HO ? 2 : 4;
    constexpr int SO = slab_ops<HO>();           // A operands per (tile, block)
    // A loads (1 KB each) per pair in eighths of the workgroup (the four
    // loading wavefronts issue twice these).
    constexpr int NA = 2 * SO / (8 * 64);
    constexpr int DA = RingDepth<F, HO>::kA, DBQ = RingDepth<F, HO>::kBQ;
    // Weight stages are loaded LB = 2 DBQ - 1 steps ahead of their first pair;
    // the first PRO steps' loads precede the first pair.
    constexpr int LB = 2 * DBQ - 1, PRO = DA > LB ? DA : LB;
    static_assert(DA >= 3 && DBQ >= 2, "ring depths");
    __shared__ SplitLds<F, HO> lds;

    const int T = tiles_m * tiles_n, L = blockIdx.x;
    const int t = (T % 8 == 0) ? (L % 8) * (T / 8) + L / 8 : L;
    const int mt = t / tiles_n, m0 = mt * kGemmBM, n0 = (t % tiles_n) * kGemmBN;

    const int tid = threadIdx.x, lane = tid & 63;
    // The wavefront index, made visibly uniform so that branches on it are scalar.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave >> 2, wm = HO ? 0 : (wave >> 1) & 1, wn = HO ? (wave & 3) : (wave & 1);
    const int li = lane & 15, g = lane >> 4;
    const int npairs = nblk >> 1;
    const uint32_t magic_v = magic_vgpr<F>();
    const size_t row_bytes = (size_t)nblk_row * F::kBytes;

    // Direct-to-LDS loads, issued by the four wavefronts of K group 0 only
    // (the same count on each, so their vmcnt moves in the same steps; K group
    // 1 issues none and computes through the loads' issue stalls: 2-3% faster
    // than spreading the loads over all eight), as buffer loads: one buffer
    // resource per operand for the workgroup's tile, a fixed per-lane offset
    // and a per-pair scalar offset, so the step's addressing is scalar work.
    // A, per pair: 2 NA (8, or 4 hi-only) 16-byte loads, 1 KB each, at entries
    // (2 NA lw + i) * 64 + lane of the slab (lw = wave % 4), whose workspace
    // order is the LDS order. B, per two pairs (every other step): NBQ 4-byte
    // loads at dword slots j * 64 + lane, j = lw + 4 r; slot t < 128 2 kDwords
    // is dword t % (2 kDwords) of the two pairs' bytes of row t / (2 kDwords),
    // higher slots re-read a valid dword into unused LDS. Two pairs per load
    // instruction put each row's 72 (or 136) contiguous bytes in one
    // instruction instead of 36 (68) in each of two: a quarter fewer weight
    // loads (9 against 12 per two Q4_0 pairs, less padding), about 1% faster.
    // The ranges of both resources fit 32 bits (K <= 2^22 on this path); each
    // ends with the segment's last block.
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(ahl + (size_t)mt * nblk_row * SO), (short)0, (int)((uint32_t)nblk * SO * 16u),
        kBufferRsrcWord3);
    const int brows = min(kGemmBN, N - n0);
    const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(w + (size_t)n0 * row_bytes), (short)0,
        (int)((brows - 1) * row_bytes + (size_t)nblk * F::kBytes), kBufferRsrcWord3);
    // Loads of a loading wavefront: NA2 A loads per pair, NBQ B loads per
    // two pairs.
    constexpr int NA2 = 2 * NA, NBQ = G::kBQLoads;
    constexpr int kDQ = 2 * G::kDwords;             // B dwords per row and stage
    const int lw = wave & 3;
    const uint32_t a_voff = (uint32_t)((lw * NA2 * 64 + lane) * 16);
    uint32_t b_voff[NBQ];
#pragma unroll
    for (int r = 0; r < NBQ; ++r) {
        const int tt = min((lw + 4 * r) * 64 + lane, G::kBQDwords - 1);
        const int row = tt / kDQ, dw = tt % kDQ;
        b_voff[r] = (uint32_t)(min(row, brows - 1) * (int)row_bytes + 4 * dw);
    }
    // Load k of a step on a loading wavefront: the NA2 A loads of pair pa,
    // then (odd steps) the NBQ B loads of pairs 2 qb and 2 qb + 1 (k is a
    // compile-time constant where this is called).
    auto issue_load = [&](int pa, int qb, int k) __attribute__((always_inline)) {
        if (k < NA2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                arsrc, (__attribute__((address_space(3))) void *)(lds.a[pa % DA] + (lw * NA2 + k) * 64),
                16, a_voff + k * 1024, (int)((uint32_t)pa * (2u * SO * 16u)), 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                brsrc, (__attribute__((address_space(3))) void *)(lds.b[(unsigned)qb % DBQ] + (lw + 4 * (k - NA2)) * 64),
                4, b_voff[k - NA2], qb * (4 * F::kBytes), 0, 0);
    };

    f32x4 acc[RM][CN];
#pragma unroll
    for (int ms = 0; ms < RM; ++ms)
#pragma unroll
        for (int ns = 0; ns < CN; ++ns)
            acc[ms][ns] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const f16 sc = (f16)0x1p-11f;
    const f16x8 scale = {sc, sc, sc, sc, sc, sc, sc, sc};

    auto run_group = [&](auto kg_c) __attribute__((always_inline)) {
        constexpr int KG = decltype(kg_c)::value;
        // Loads per step of this wavefront (even steps: A only; odd steps: A
        // and B): all of the workgroup's on K group 0's four, none on K group
        // 1's.
        constexpr int NAK = KG == 0 ? NA2 : 0, NBK = KG == 0 ? NBQ : 0;
        // B of column group ns, block 2p + KG: the row's raw pair bytes hold block
        // KG at byte kBytes KG. KG is a compile-time constant (the loop exists
        // once per K group), so the realignment (where the quant bytes straddle
        // dwords) and the half of the dword that holds d are fixed per loop.
        struct BCol {
            QsRaw<F, KG> qs;
            uint32_t dw;
        };
        auto read_b = [&](const uint32_t *bstage, int ns) __attribute__((always_inline)) {
            const uint32_t *rb = bstage + (wn * (CN * 16) + ns * 16 + li) * kDQ;
            return BCol{read_qs_raw<F, KG>(rb, g), rb[d_dword<F, KG>()]};
        };
        // The operands of one pair held in registers: the A operands of the
        // wavefront's RM row groups and the raw B bytes of its CN column
        // groups.
        struct Ops {
            f16x8 hi[RM], lo[HO ? 1 : RM];
            BCol b[CN];
        };
        // Part i of pair q's operands (row groups i RM/CN .. (i+1) RM/CN - 1,
        // column group i).
        auto read_ops = [&](int q, Ops &o, int i) __attribute__((always_inline)) {
            const u32x4 *ap = lds.a[q % DA] + KG * SO + wm * RM * 64 + lane;
#pragma unroll
            for (int r = i * (RM / CN); r < (i + 1) * (RM / CN); ++r) {
                o.hi[r] = bitcast<f16x8>(ap[r * 64]);
                if constexpr (!HO)
                    o.lo[r] = bitcast<f16x8>(ap[8 * 64 + r * 64]);
            }
            o.b[i] = read_b(lds.b[((unsigned)q >> 1) % DBQ] + (q & 1) * G::kDwords, i);
        };
        // LDS reads of one part.
        constexpr int kDsReads = (RM / CN) * (HO ? 1 : 2) + QsRaw<F, KG>::n + 1;

        // Software pipeline over the four column groups of a pair: the MFMAs of
        // group ns are issued between the scale FMAs of group ns - 1 (whose results
        // are ready) and the decode of group ns + 1. Group results alternate
        // between two register sets by the parity of ns, and the group before
        // group 0 is group 3 of the previous pair (zeros before the first pair),
        // so every index is a compile-time constant.
        f32x4 cbuf[2][RM];
        float dbuf[2] = {0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ms = 0; ms < RM; ++ms)
                cbuf[h][ms] = zero4;
        struct BOps {
            f16x8 q, s;   // the codes (x 2^kHiLog2 in slots 4..7) and the same times 2^-11
            float d;
        };
        auto decode_b = [&](const BCol &bc) __attribute__((always_inline)) {
            uint32_t x[F::kQsDwords];
            align_qs<F, KG>(bc.qs, x);
            BOps o;
            o.d = f16_bits_to_f32(d_from_dword<F, KG>(bc.dw));
            o.q = F::decode(x, magic_v);
            if constexpr (!HO)
                o.s = o.q * scale;
            return o;
        };
        // One scheduling region per column group ns: its eight MFMAs (the four lo
        // products, then the four hi products that add onto them) interleaved
        // with the scale FMAs of group ns - 1, the decode of group ns + 1 and
        // part ns of the next pair's operands (LDS reads that land during this
        // pair's MFMAs, so no step starts by waiting on LDS). The scheduling-group
        // barriers ask for one MFMA, one LDS read while any remain, then four VALU
        // instructions, eight times per region; hard barriers between regions
        // keep that order.
        auto compute_pair = [&](auto odd_c, const Ops &cur_ops, Ops &next_ops, int next_pair,
                                int dma_a, int dma_b) __attribute__((always_inline)) {
            constexpr int NLK = NAK + (decltype(odd_c)::value ? NBK : 0);
            BOps cur = decode_b(cur_ops.b[0]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ns = 0; ns < CN; ++ns) {
                f32x4 *c = cbuf[ns & 1];
                const f32x4 *cp = cbuf[(ns + 1) & 1];      // group ns - 1 (mod CN; CN is even)
                const float dp = dbuf[(ns + 1) & 1];
                // The two-term form multiplies the small lo terms first and adds
                // the hi products onto them (the rounding of the lo chain then
                // acts on sums 2^-11 the size of the hi ones).
#pragma unroll
                for (int ms = 0; ms < RM; ++ms) {
                    if constexpr (HO)
                        c[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur_ops.hi[ms], cur.q, zero4, 0, 0, 0);
                    else
                        c[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur_ops.lo[ms], cur.s, zero4, 0, 0, 0);
                }
                read_ops(next_pair, next_ops, ns);
                // The step's loads go out spread over the four regions (loads
                // [NLK ns / 4, NLK (ns + 1) / 4), rounded up) and, within a region,
                // between MFMAs, so the address unit works while the matrix cores
                // do and no wavefront's MFMAs queue behind a load. They write LDS,
                // so they follow this region's LDS reads in program order (the
                // compiler keeps LDS accesses it cannot tell apart in order).
#pragma unroll
                for (int k = (NLK * ns + CN - 1) / CN; k < (NLK * (ns + 1) + CN - 1) / CN; ++k)
                    issue_load(dma_a, dma_b, k);
                const int np = (ns + CN - 1) % CN;
#pragma unroll
                for (int ms = 0; ms < RM; ++ms)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[ms][np][q] = fmaf(dp, cp[ms][q], acc[ms][np][q]);
                // Pin these FMAs to this region: IR passes would otherwise sink
                // them past the scheduling barriers, to the end of the pair.
                if constexpr (RM == 4)
                    asm volatile("" : "+v"(acc[0][np]), "+v"(acc[1][np]), "+v"(acc[2][np]), "+v"(acc[3][np]));
                else
                    asm volatile("" : "+v"(acc[0][np]), "+v"(acc[1][np]), "+v"(acc[2][np]), "+v"(acc[3][np]),
                                      "+v"(acc[4][np]), "+v"(acc[5][np]), "+v"(acc[6][np]), "+v"(acc[7][np]));
                BOps nxt = cur;
                if (ns + 1 < CN)
                    nxt = decode_b(cur_ops.b[ns + 1]);
                if constexpr (!HO) {
#pragma unroll
                    for (int ms = 0; ms < RM; ++ms)
                        c[ms] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur_ops.hi[ms], cur.q, c[ms], 0, 0, 0);
                }
                dbuf[ns & 1] = cur.d;
                // Eight MFMAs per region, each followed by LDS reads while any
                // remain, the region's loads towards its end, and its share of
                // the VALU work.
                constexpr int NM = RM * (HO ? 1 : 2);
                constexpr int kDsPerSlot = (kDsReads + NM - 1) / NM;
                constexpr int kValuPerSlot = HO ? (F::kBytes == kQ4Bytes ? 7 : 6) : 4;
                constexpr int kRegionLoads = (NLK + CN - 1) / CN;   // at most, per region
                const int nl = (NLK * (ns + 1) + CN - 1) / CN - (NLK * ns + CN - 1) / CN;
#pragma unroll
                for (int u = 0; u < NM; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    if (u * kDsPerSlot < kDsReads)
                        __builtin_amdgcn_sched_group_barrier(0x100, kDsPerSlot, 0);   // LDS reads
                    if (u >= NM - nl && u >= NM - kRegionLoads)
                        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // one load
                    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerSlot, 0);   // VALU
                }
                __builtin_amdgcn_sched_barrier(0);
                cur = nxt;
            }
        };

        // Ring schedule: step p issues the A loads of pair p + DA and, when p is
        // odd, then the B loads of pairs p + LB and p + LB + 1 (double stage
        // Q = (p + LB) / 2, in B stage Q % DBQ). Pair q's A slab goes to A
        // stage q % DA during step q - DA, its B bytes to B stage (q / 2) % DBQ
        // during step 2 (q / 2) - LB (q - LB or q - LB - 1). Both are complete
        // by the barrier ending step q - 2, are read into registers during
        // step q - 1, and pair q is computed in step q. An A stage is loaded
        // again in step q (pair q + DA), after the barrier that ends step
        // q - 1, by which every wavefront has read it; B stage Q % DBQ again
        // in step 2 Q + 1, after the barrier ending step 2 Q, by which pair
        // 2 Q + 1's bytes are read. Loads complete in issue order, so at the
        // barrier ending step p the loads issued after the last one pair p + 2
        // needs may still be in flight: ring_in_flight counts them, one count
        // for even and one for odd p (near the end, where fewer are issued, the
        // barrier waits for everything). The last step reads stages no load is
        // writing any more, and discards what it read.
        constexpr int kInFlightEven = ring_in_flight(0, DA, LB, NAK, NBK);
        constexpr int kInFlightOdd = ring_in_flight(1, DA, LB, NAK, NBK);
        static_assert(kInFlightEven < 64 && kInFlightOdd < 64, "vmcnt counts to 63");
        // The loads of steps -PRO .. -1, in the order those steps would issue
        // them (a step before the first A load issues only its B loads). A step whose
        // pair is past the last one reloads the last pair (or two) into its own
        // stage (the same bytes), so every step issues its count of loads and,
        // with at least PRO pairs, every barrier can count them; shorter problems
        // wait for all. K group 1 has no loads of its own in flight: its
        // barriers only order, and wait for the loaders, which wait for theirs
        // before the barrier.
        const bool counted = npairs >= PRO;
        const int last = npairs - 1, lastq = last >> 1;
        for (int t = -PRO; t < 0; ++t) {
#pragma unroll
            for (int k = 0; k < NAK + NBK; ++k)
                if (k < NAK ? t + DA >= 0 : (t & 1) != 0)
                    issue_load(min(t + DA, last), min((t + LB) / 2, lastq), k);
        }
        if (counted)
            ring_barrier<kInFlightOdd>();   // pairs 0 and 1 complete
        else
            ring_barrier<0>();
        Ops O0, O1;
#pragma unroll
        for (int i = 0; i < CN; ++i)
            read_ops(0, O0, i);
        // Step 0 reloads A stage 0: every wavefront must have read pair 0's
        // operands first.
        if (counted)
            ring_barrier<kInFlightOdd>();
        else
            ring_barrier<0>();
        auto step = [&](auto odd_c, int p, const Ops &cur_ops, Ops &next_ops) __attribute__((always_inline)) {
            constexpr bool odd = decltype(odd_c)::value;
            compute_pair(odd_c, cur_ops, next_ops, p + 1, min(p + DA, last), min((p + LB) / 2, lastq));
            if (counted)
                ring_barrier<odd ? kInFlightOdd : kInFlightEven>();   // pair p + 2 complete
            else
                ring_barrier<0>();
        };
        for (int p = 0; p < npairs; p += 2) {
            step(std::false_type{}, p, O0, O1);
            if (p + 1 < npairs)
                step(std::true_type{}, p + 1, O1, O0);
        }
        // FMAs of the last column group (group CN - 1 of the last pair, in set 1).
#pragma unroll
        for (int ms = 0; ms < RM; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[ms][CN - 1][q] = fmaf(dbuf[1], cbuf[1][ms][q], acc[ms][CN - 1][q]);
    };
    if (kg == 0)
        run_group(std::integral_constant<int, 0>{});
    else
        run_group(std::integral_constant<int, 1>{});

    // Group 1 hands its partial tile to group 0 through LDS (every load has
    // landed and every wavefront has passed the last barrier):
    // [wavefront of the group][value][lane].
    float *red = reinterpret_cast<float *>(&lds.a[0][0]);
    static_assert(sizeof(lds.a) >= 4 * 64 * 64 * sizeof(float), "reduction buffer");
    const int wq = wave & 3;
    if (kg == 1) {
#pragma unroll
        for (int ms = 0; ms < RM; ++ms)
#pragma unroll
            for (int ns = 0; ns < CN; ++ns)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[(wq * 64 + ms * (CN * 4) + ns * 4 + q) * 64 + lane] = acc[ms][ns][q];
    }
    __syncthreads();
    if (kg == 0) {
        // Lane (li, g) of tile (ms, ns) holds rows 4g..4g+3 of column li.
        // Offsets are 32-bit (M N < 2^31 on this path, checked at launch).
        // Rows of scaled activations (every form that passes row exponents)
        // are scaled back by 2^-row_exp[m]; a later K segment adds its part to
        // what the earlier ones left in y.
        const bool scaled_rows = HO || row_exp != nullptr;
        const int mb = m0 + wm * (RM * 16) + 4 * g, nb = n0 + wn * (CN * 16) + li;
#pragma unroll
        for (int ms = 0; ms < RM; ++ms) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = mb + ms * 16 + q;
                const uint32_t row_off = (uint32_t)m * (uint32_t)N + (uint32_t)nb;
                int pe = 0;
                if (scaled_rows && m < M)
                    pe = row_exp[m];
#pragma unroll
                for (int ns = 0; ns < CN; ++ns) {
                    float v = acc[ms][ns][q] + red[(wq * 64 + ms * (CN * 4) + ns * 4 + q) * 64 + lane];
                    if (scaled_rows)
                        v = ldexpf(v, -pe);
                    if (m < M && nb + ns * 16 < N) {
                        if (accumulate)
                            v += y[row_off + ns * 16];
                        y[row_off + ns * 16] = v;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bfloat16 activations. A bfloat16 value has an 8-bit significand, so once its
// row is scaled by a power of two 2^p that brings the row's largest magnitude
// into [2^15, 2^16), every element within 2^32 of that maximum (2^28 on Q4_0's
// slots 4..7, which carry a further 2^-4) is exactly a binary16 number: one f16
// term per activation replaces the hi / lo pair of the f32 path, and the same
// MFMAs on the same weight decode give products that are exact in f32. The
// result row is scaled back by 2^-p in the epilogue (exact unless it lands in
// the f32 subnormal range). Smaller elements round to the binary16 grid (2^-24
// after scaling, 2^(E - 39) in the row's own units for max |a| in [2^E,
// 2^(E+1))).
//
// * The row's exponent: the largest magnitude is the largest bfloat16 bit
//   pattern with the sign cleared (which orders finite values by magnitude),
//   and p = 15 - E; p = 0 for an all-zero row or one that holds an infinity
//   or NaN.
// * k_row_exp_bf16 (general kernel's shapes): one wavefront per row, all of
//   its loads in flight at once.
// * k_gemm_prep_bf16 (split path): the exponents and the operands in one
//   launch, arranged as k_gemm_prep_f32 (a workgroup per 16-row group and K
//   part, each finding its group's exponents over the whole rows), writing
//   only the hi operand: operand [mt][kb][sub][lane] in the format's slot
//   order, rows past M zero. (One workgroup per 16-row group, without the K
//   parts, was measured slower: at M = 1024 it leaves three quarters of the
//   CUs idle.)
// * k_gemm_prep_bf16_f32 (general kernel's shapes): the scaled activations as
//   f32, row-major (f16(a') is then exact and the lo term 0).

constexpr int kRowExpWaves = 4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Largest |a| of row `row` (K bfloat16 values, K % 32 == 0) as a cleared-sign
// bit pattern, in every lane of the wavefront.
__device__ __forceinline__ uint32_t row_max_bits_bf16(const uint16_t *__restrict__ row, int K,
                                                      int lane)
{
    // A row is a whole number of 64-byte lines, read 16 bytes a lane.
    const uint4 *r4 = reinterpret_cast<const uint4 *>(row);
    uint32_t mx = 0;
#pragma unroll 8
    for (int i = lane; i < K / 8; i += 64) {
        const uint4 v = r4[i];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            mx = max(mx, max(w4[j] & 0x7FFFu, (w4[j] >> 16) & 0x7FFFu));
    }
    return wave_max_u32(mx);
}

// p = 15 - E for a largest magnitude in [2^E, 2^(E+1)); 0 for zero or non-finite.
__device__ __forceinline__ int row_exp_from_bits(uint32_t mx)
{
    if (mx == 0 || mx >= 0x7F80u)
        return 0;
    const int ef = (int)(mx >> 7);
    // Subnormals are (mantissa) 2^-133.
    const int E = ef > 0 ? ef - 127 : (31 - __builtin_clz(mx)) - 133;
    return 15 - E;
}

__global__ __launch_bounds__(64 * kRowExpWaves) void k_row_exp_bf16(const uint16_t *__restrict__ a,
                                                                   int *__restrict__ row_exp,
                                                                   int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * kRowExpWaves + (threadIdx.x >> 6);
    if (m >= M)   // whole wavefronts only
        return;
    const int p = row_exp_from_bits(row_max_bits_bf16(a + (size_t)m * K, K, lane));
    if (lane == 0)
        row_exp[m] = p;
}

// Blocks a wavefront of k_gemm_prep_bf16 takes at a time (the split path has
// an even number of blocks per row): each row's segment is a whole 128-byte
// line.
constexpr int kPrepBlocks = 2;

template <class F>
__device__ __forceinline__ void prep_bf16_pair(const uint16_t *__restrict__ a, int p,
                                               u32x4 *__restrict__ ops, int M, int K, long long R,
                                               int kb0, int lane)
{
    const int nblk = K >> 5;
    const int li = lane & 15, g = lane >> 4;
    const long long m = R * 16 + li;
    f16x8 hi[kPrepBlocks] = {};
    if (m < M) {
        const uint16_t *blk0 = a + m * K + (long long)kb0 * 32;
        uint2 L[kPrepBlocks], H[kPrepBlocks];
#pragma unroll
        for (int u = 0; u < kPrepBlocks; ++u) {
            L[u] = *reinterpret_cast<const uint2 *>(blk0 + u * 32 + F::a_lo(g));
            H[u] = *reinterpret_cast<const uint2 *>(blk0 + u * 32 + F::a_hi(g));
        }
        const int ph = p - F::kHiLog2;   // slots 4..7 carry a further 2^-kHiLog2
#pragma unroll
        for (int u = 0; u < kPrepBlocks; ++u) {
            // Elements 0..3 of a group are the low and high halves of two
            // dwords, in the slot order x, z, y, w of the f32 path.
            const float e[8] = {
                ldexpf(bf16_bits_to_f32(L[u].x & 0xFFFFu), p), ldexpf(bf16_bits_to_f32(L[u].y & 0xFFFFu), p),
                ldexpf(bf16_bits_to_f32(L[u].x >> 16), p),     ldexpf(bf16_bits_to_f32(L[u].y >> 16), p),
                ldexpf(bf16_bits_to_f32(H[u].x & 0xFFFFu), ph), ldexpf(bf16_bits_to_f32(H[u].y & 0xFFFFu), ph),
                ldexpf(bf16_bits_to_f32(H[u].x >> 16), ph),    ldexpf(bf16_bits_to_f32(H[u].y >> 16), ph)};
#pragma unroll
            for (int s = 0; s < 8; ++s)
                hi[u][s] = (f16)e[s];
        }
    }
    u32x4 *dst = ops + ((R >> 3) * nblk + kb0) * slab_ops<true>() + (R & 7) * 64 + lane;
#pragma unroll
    for (int u = 0; u < kPrepBlocks; ++u)
        dst[u * slab_ops<true>()] = bitcast<u32x4>(hi[u]);
}

// The bfloat16 split path's preparation in one launch, arranged as
// k_gemm_prep_f32: workgroup (R, q) finds the 16 rows' exponents of group R
// over the whole rows (one row per wavefront; part 0 writes row_exp), then
// its wavefronts take the pairs of blocks of K part q in turn. Each pair:
// lane (g, li) reads row li's slots of lane group g for both blocks and
// writes their binary16 values (row past M: zeros) in slab order.
template <class F>
__global__ __launch_bounds__(64 * kPrepWaves) void k_gemm_prep_bf16(const uint16_t *__restrict__ a,
                                                                  int *__restrict__ row_exp,
                                                                  u32x4 *__restrict__ ops, int M,
                                                                  int K, int part_blocks)
{
    __shared__ int s_p[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long R = blockIdx.x;
    const int nblk = K >> 5;
    const int kb0 = (int)blockIdx.y * part_blocks, kb1 = min(kb0 + part_blocks, nblk);
    static_assert(kPrepWaves == 16, "one row of the group per wavefront");
    const long long m = R * 16 + wave;
    int pw = 0;
    if (R * 16 < M)
        pw = row_exp_from_bits(row_max_bits_bf16(a + min(m, (long long)M - 1) * K, K, lane));
    if (lane == 0) {
        s_p[wave] = pw;
        if (blockIdx.y == 0 && m < M)
            row_exp[m] = pw;
    }
    __syncthreads();
    const int p = s_p[lane & 15];
    for (int kb = kb0 + kPrepBlocks * wave; kb < kb1; kb += kPrepBlocks * kPrepWaves)
        prep_bf16_pair<F>(a, p, ops, M, K, R, kb, lane);
}

__global__ __launch_bounds__(256) void k_gemm_prep_bf16_f32(const uint16_t *__restrict__ a,
                                                           const int *__restrict__ row_exp,
                                                           float4 *__restrict__ out, int K,
                                                           long long n_quads)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_quads)
        return;
    const int p = row_exp[(i * 4) / K];   // K % 32 == 0: a quad never straddles rows
    const uint2 v = reinterpret_cast<const uint2 *>(a)[i];
    out[i] = make_float4(ldexpf(bf16_bits_to_f32(v.x & 0xFFFFu), p),
                         ldexpf(bf16_bits_to_f32(v.x >> 16), p),
                         ldexpf(bf16_bits_to_f32(v.y & 0xFFFFu), p),
                         ldexpf(bf16_bits_to_f32(v.y >> 16), p));
}

// ---------------------------------------------------------------------------
// f32 activations: the row exponents. k_row_exp_f32 (one wavefront per row)
// takes the largest |a| of the row as the largest f32 bit pattern with the
// sign cleared (which orders finite values by magnitude) and sets p = 14 - E
// for a largest magnitude in [2^E, 2^(E+1)); 0 for an all-zero row or one
// that holds an infinity or NaN.

// Largest |a| of row `row` (K f32 values, K % 32 == 0, 16-byte aligned) as a
// cleared-sign bit pattern, in every lane of the wavefront. Sixteen 16-byte
// loads per lane per round are issued before any is used (a 4096-element row
// in one round), so a compute unit keeps enough bytes in flight even with one
// wavefront per row.
__device__ __forceinline__ uint32_t row_max_bits_f32(const float *__restrict__ row, int K, int lane)
{
    const uint4 *r4 = reinterpret_cast<const uint4 *>(row);
    uint32_t mx = 0;
#pragma unroll 16
    for (int i = lane; i < K / 4; i += 64) {
        const uint4 v = r4[i];
        mx = max(mx, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu),
                         max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
    return wave_max_u32(mx);
}

// The row's power of two from its largest cleared-sign bit pattern.
__device__ __forceinline__ int row_exp_from_bits_f32(uint32_t mx)
{
    int p = 0;
    if (mx != 0 && mx < 0x7F800000u) {
        const int ef = (int)(mx >> 23);
        // Subnormals are (mantissa) 2^-149.
        const int E = ef > 0 ? ef - 127 : (31 - __builtin_clz(mx)) - 149;
        p = 14 - E;
    }
    return p;
}

__global__ __launch_bounds__(64 * kRowExpWaves) void k_row_exp_f32(const float *__restrict__ a,
                                                                  int *__restrict__ row_exp,
                                                                  int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * kRowExpWaves + (threadIdx.x >> 6);
    if (m >= M)   // whole wavefronts only
        return;
    const int p = row_exp_from_bits_f32(row_max_bits_f32(a + (size_t)m * K, K, lane));
    if (lane == 0)
        row_exp[m] = p;
}

// The split path's preparation in one launch: the row exponents and the
// two-term operands (the same values as k_row_exp_f32 and a split per block).
// Workgroup (R, q) takes 16-row group R and K part q (blocks [q L, q L + L)).
// Every element of a row bounds its exponent, so each of a row group's
// workgroups first finds the 16 rows' maxima over the whole row itself (the
// rows stay in L2 after the first reads; repeating the maxima avoids a
// grid-wide dependency), one row per wavefront; part 0 writes them to
// row_exp. Then its sixteen wavefronts split the part's blocks in turn, two
// at a time.

template <class F>
__global__ __launch_bounds__(64 * kPrepWaves) void k_gemm_prep_f32(const float *__restrict__ a,
                                                                 int *__restrict__ row_exp,
                                                                 u32x4 *__restrict__ ahl, int M,
                                                                 int K, int part_blocks)
{
    __shared__ float4 tile[kPrepWaves][16 * 9];
    __shared__ int s_p[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long R = blockIdx.x;
    const int nblk = K >> 5;
    const int kb0 = (int)blockIdx.y * part_blocks, kb1 = min(kb0 + part_blocks, nblk);
    // Row `wave` of the group (a group wholly past M, part of the last tile,
    // needs no exponents: its operands are zeros).
    static_assert(kPrepWaves == 16, "one row of the group per wavefront");
    const long long m = R * 16 + wave;
    int pw = 0;
    if (R * 16 < M)
        pw = row_exp_from_bits_f32(row_max_bits_f32(a + min(m, (long long)M - 1) * K, K, lane));
    if (lane == 0) {
        s_p[wave] = pw;
        if (blockIdx.y == 0 && m < M)
            row_exp[m] = pw;
    }
    __syncthreads();
    const int p = s_p[lane & 15];
    float4 *t = tile[wave];
    int kb = kb0 + wave;
    for (; kb + kPrepWaves < kb1; kb += 2 * kPrepWaves) {
        const SplitRows x0 = split_load(a, M, K, R, kb, lane);
        const SplitRows x1 = split_load(a, M, K, R, kb + kPrepWaves, lane);
        split_store<F>(x0, p, ahl, M, nblk, R, kb, t, lane);
        split_store<F>(x1, p, ahl, M, nblk, R, kb + kPrepWaves, t, lane);
    }
    if (kb < kb1)
        split_store<F>(split_load(a, M, K, R, kb, lane), p, ahl, M, nblk, R, kb, t, lane);
}

// Longest run of block partials that one accumulator adds in sequence in a
// launch. Longer K is cut into segments, one launch each, every launch after
// the first adding its part into y; see the summation order at the top.
constexpr int kMaxChain = 112;

struct KSegments {
    int n, len;   // n segments of len blocks (the last one the rest)
};

// per_term: blocks per term of an accumulator's chain, 2 on the split kernel
// (its two K groups take alternate blocks), 1 on the general kernel.
static KSegments k_segments(int nblk, int per_term)
{
    const int terms = (nblk + per_term - 1) / per_term;
    const int n = (terms + kMaxChain - 1) / kMaxChain;
    const int len = (terms + n - 1) / n * per_term;
    return {(nblk + len - 1) / len, len};
}

template <class F, bool HO>
static hipError_t launch_split_segments(const u32x4 *ops, const uint8_t *w, float *y, int M, int N,
                                        int K, int tiles_m, int tiles_n, const int *row_exp,
                                        hipStream_t s)
{
    const int nblk = K >> 5;
    const KSegments sg = k_segments(nblk, 2);
    const unsigned T = (unsigned)tiles_m * (unsigned)tiles_n;
    for (int i = 0; i < sg.n; ++i) {
        const int kb0 = i * sg.len, nb = min(sg.len, nblk - kb0);
        const hipError_t e = launch_kernel(
            k_gemm_split<F, HO>, dim3(T), dim3(kSplitGemmThreads), 0, s,
            ops + (size_t)kb0 * slab_ops<HO>(), w + (size_t)kb0 * F::kBytes, y, M, N, nblk, nb,
            tiles_m, tiles_n, row_exp, i > 0 ? 1 : 0);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <class F>
static hipError_t launch_any_segments(const float *a, const uint8_t *w, float *y, int M, int N,
                                      int K, int tiles_m, int tiles_n, const int *row_exp,
                                      int scale_in, hipStream_t s)
{
    const int nblk = K >> 5;
    const KSegments sg = k_segments(nblk, 1);
    const unsigned T = (unsigned)tiles_m * (unsigned)tiles_n;
    for (int i = 0; i < sg.n; ++i) {
        const int kb0 = i * sg.len, nb = min(sg.len, nblk - kb0);
        const hipError_t e = launch_kernel(k_gemm_any<F>, dim3(T), dim3(kGemmThreads), 0, s,
                                           a + (size_t)kb0 * 32, w + (size_t)kb0 * F::kBytes, y,
                                           M, N, K, nb, tiles_m, tiles_n, row_exp, scale_in,
                                           i > 0 ? 1 : 0);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// workspace: the row exponents (q4v::gemm_row_exp_bytes(M)), then on the split
// path (split: the caller's choice, q4v::gemm_splits_activations(K) with
// M N < 2^31) the two-term operands.
template <class F>
static hipError_t launch_gemm_f(const float *a, const uint8_t *w, float *y, int M, int N, int K,
                                void *workspace, hipStream_t s, bool split)
{
    const int tiles_m = (M + kGemmBM - 1) / kGemmBM, tiles_n = (N + kGemmBN - 1) / kGemmBN;
    const long long T = (long long)tiles_m * tiles_n;
    if (T > 0x7fffffffLL)
        return hipErrorInvalidValue;
    int *row_exp = static_cast<int *>(workspace);
    if (!split) {
        const hipError_t e = launch_kernel(
            k_row_exp_f32, dim3((unsigned)((M + kRowExpWaves - 1) / kRowExpWaves)),
            dim3(64 * kRowExpWaves), 0, s, a, row_exp, M, K);
        if (e != hipSuccess)
            return e;
        return launch_any_segments<F>(a, w, y, M, N, K, tiles_m, tiles_n, row_exp, 1, s);
    }
    u32x4 *ahl = reinterpret_cast<u32x4 *>(static_cast<char *>(workspace) +
                                           q4v::gemm_row_exp_bytes(M));
    // Row groups of every tile (those past M get zero operands).
    const long long groups = (long long)tiles_m * 8;
    const int nblk = K / 32;
    const int part_blocks = prep_part_blocks(groups, nblk, 1);
    const unsigned qn = (unsigned)((nblk + part_blocks - 1) / part_blocks);
    if (groups > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const hipError_t e = launch_kernel(k_gemm_prep_f32<F>, dim3((unsigned)groups, qn),
                                       dim3(64 * kPrepWaves), 0, s, a, row_exp, ahl, M, K,
                                       part_blocks);
    if (e != hipSuccess)
        return e;
    return launch_split_segments<F, false>(ahl, w, y, M, N, K, tiles_m, tiles_n, row_exp, s);
}

template <class F>
static hipError_t launch_gemm_bf16_f(const uint16_t *a, const uint8_t *w, float *y, int M, int N,
                                     int K, void *workspace, hipStream_t s)
{
    const int tiles_m = (M + kGemmBM - 1) / kGemmBM, tiles_n = (N + kGemmBN - 1) / kGemmBN;
    const long long T = (long long)tiles_m * tiles_n;
    if (T > 0x7fffffffLL)
        return hipErrorInvalidValue;
    int *row_exp = static_cast<int *>(workspace);
    void *act = static_cast<char *>(workspace) + q4v::gemm_row_exp_bytes(M);
    hipError_t e;
    if (!q4v::gemm_bf16_splits(M, N, K)) {
        e = launch_kernel(k_row_exp_bf16, dim3((unsigned)((M + kRowExpWaves - 1) / kRowExpWaves)),
                          dim3(64 * kRowExpWaves), 0, s, a, row_exp, M, K);
        if (e != hipSuccess)
            return e;
        const long long n_quads = (long long)M * K / 4;
        const long long grid = (n_quads + 255) / 256;
        if (grid > 0x7fffffffLL)
            return hipErrorInvalidValue;
        e = launch_kernel(k_gemm_prep_bf16_f32, dim3((unsigned)grid), dim3(256), 0, s, a,
                          (const int *)row_exp, static_cast<float4 *>(act), K, n_quads);
        if (e != hipSuccess)
            return e;
        return launch_any_segments<F>((const float *)act, w, y, M, N, K, tiles_m, tiles_n,
                                      row_exp, 0, s);
    }
    // Every 16-row group of the padded tiles (groups past M write zeros), in
    // K parts of whole pairs.
    const long long groups = (long long)tiles_m * 8;
    const int part_blocks = prep_part_blocks(groups, K / 32, kPrepBlocks);
    if (groups > 0x7fffffffLL)
        return hipErrorInvalidValue;
    e = launch_kernel(k_gemm_prep_bf16<F>,
                      dim3((unsigned)groups, (unsigned)((K / 32 + part_blocks - 1) / part_blocks)),
                      dim3(64 * kPrepWaves), 0, s, a, row_exp, static_cast<u32x4 *>(act), M, K,
                      part_blocks);
    if (e != hipSuccess)
        return e;
    return launch_split_segments<F, true>((const u32x4 *)act, w, y, M, N, K, tiles_m, tiles_n,
                                          row_exp, s);
}

// The split kernel stores with 32-bit offsets: M N < 2^31 on its path.
static bool gemm_f32_splits(int M, int N, int K)
{
    return q4v::gemm_splits_activations(K) && (long long)M * N < (1LL << 31);
}

hipError_t launch_gemm(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M, int N,
                       int K, void *workspace, hipStream_t s)
{
    const bool split = gemm_f32_splits(M, N, K);
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemm_f<FmtQ8_0>(a, w, y, M, N, K, workspace, s, split);
    return launch_gemm_f<FmtQ4_0>(a, w, y, M, N, K, workspace, s, split);
}

// ---------------------------------------------------------------------------
// The f32 GEMM with no workspace argument (q4_gemm, q8_gemm): for callers that
// cannot allocate. Its scratch, the row exponents and two-term operands of one
// chunk of rows, is this file-scope device array, which every GPU the library
// runs on holds (its own copy) until the process ends. On the host the array's
// name denotes a host-side stand-in, not device memory, so host code uses only
// the address hipGetSymbolAddress returns for the device a call runs on,
// looked up once per device (with that device current) and kept.
//
// Rows are taken in chunks whose workspace fits the array: multiples of 128
// rows on the split path, so every 128-row tile computes exactly what it would
// in one launch over all rows (the result equals q4_gemm_ws's bit for bit).
// Every kernel writes the scratch it reads before reading it, so nothing has to
// start at zero; calls that overlap in time on one GPU share the array and
// race.
static __device__ __align__(256) uint8_t scratch[kGemmScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex scratch_mu;
std::atomic<void *> scratch_ptr[kScratchDevices];
}  // namespace

// The device address of `scratch` on the device of stream s (the current
// device for the null stream).
static hipError_t scratch_address(hipStream_t s, void **out)
{
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    void *p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = 0;
            if ((e = hipGetDevice(&cur)) != hipSuccess)
                return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
                return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t back = hipSetDevice(cur);
                if (e == hipSuccess)
                    e = back;
            }
            if (e != hipSuccess || !p)
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_gemm_noalloc(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M,
                               int N, int K, hipStream_t s)
{
    void *scr = nullptr;
    hipError_t e = scratch_address(s, &scr);
    if (e != hipSuccess)
        return e;
    bool split = gemm_f32_splits(M, N, K);
    long long rows = 0;
    if (split) {
        // q4v::gemm_workspace_bytes(R, N, K) = pad256(4 R) + R K 4 for R a
        // multiple of 128 (<= 256 + R (K 4 + 4)).
        rows = (long long)((kGemmScratchBytes - 256) / ((size_t)K * 4 + 4)) / kGemmBM * kGemmBM;
        if (rows < kGemmBM)
            split = false;   // K too long for one tile of operands: the general kernel
    }
    if (!split)
        rows = (long long)(kGemmScratchBytes / 4) / 256 * 256;   // the row exponents only
    for (long long r0 = 0; r0 < M; r0 += rows) {
        const int rc = (int)(M - r0 < rows ? M - r0 : rows);
        const float *ac = a + r0 * K;
        float *yc = y + r0 * N;
        e = fmt == WeightFormat::kQ8_0
                ? launch_gemm_f<FmtQ8_0>(ac, w, yc, rc, N, K, scr, s, split)
                : launch_gemm_f<FmtQ4_0>(ac, w, yc, rc, N, K, scr, s, split);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_gemm_bf16(WeightFormat fmt, const uint16_t *a, const uint8_t *w, float *y, int M,
                            int N, int K, void *workspace, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemm_bf16_f<FmtQ8_0>(a, w, y, M, N, K, workspace, s);
    return launch_gemm_bf16_f<FmtQ4_0>(a, w, y, M, N, K, workspace, s);
}

// ---------------------------------------------------------------------------
// Q8_0-quantized activations (a_q: the [M, K/32] Q8_0 block stream, row m's
// blocks contiguous in K order). A dequantized activation q d is an 8-bit code
// times an 11-bit binary16 scale, exact in f32 with at most 18 significant
// bits; the two-term split of the f32 path (hi = f16(v), lo = f16((v - hi)
// 2^11)) holds any such value exactly while it stays inside binary16's range,
// so the f32 GEMM kernels run unchanged on operands made from the blocks.
// * Range: a Q8_0 block can hold up to 128 x 65504 in magnitude. Each row is
//   scaled by the power of two 2^p that puts 128 max_b |d_b| (an upper bound
//   of the row's magnitudes) in [2^14, 2^15), p = 7 - E for the largest |d| in
//   [2^E, 2^(E+1)) (0 for an all-zero row). The scaled values stay below 2^15
//   and the epilogue scales each result row back by 2^-p.
// * row_exp_q8a: one wavefront per row, the largest |d| as the largest
//   binary16 bit pattern with the sign cleared (k_row_exp_q8a off the split
//   path).
// * k_gemm_prep_q8a (split path): the exponents and the split in one launch,
//   arranged as k_gemm_prep_f32; split_q8_block splits as the f32 path
//   (split_store) from the blocks: code q, d 2^p, the product exact in f32,
//   then the same split and operand order.
// * Off the split path: k_q8a_to_f32 writes the scaled values as f32 for
//   k_gemm_any (which takes the same row exponents).

// The exponent of row `row` (nblk Q8_0 blocks), in every lane of the wavefront.
__device__ __forceinline__ int row_exp_q8a(const uint8_t *__restrict__ row, int nblk, int lane)
{
    uint32_t mx = 0;
    for (int b = lane; b < nblk; b += 64)
        mx = max(mx, load_u16(row + (size_t)b * kQ8Bytes) & 0x7FFFu);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    int p = 0;
    if (mx != 0 && mx < 0x7C00u) {
        const int ef = (int)(mx >> 10);
        // Subnormal binary16 scales are (mantissa) 2^-24.
        const int E = ef > 0 ? ef - 15 : (31 - __builtin_clz(mx)) - 24;
        p = 7 - E;
    }
    return p;
}

__global__ __launch_bounds__(64 * kRowExpWaves) void k_row_exp_q8a(const uint8_t *__restrict__ aq,
                                                                  int *__restrict__ row_exp, int M,
                                                                  int K)
{
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * kRowExpWaves + (threadIdx.x >> 6);
    if (m >= M)   // whole wavefronts only
        return;
    const int nblk = K >> 5;
    const int p = row_exp_q8a(aq + (size_t)m * (size_t)nblk * kQ8Bytes, nblk, lane);
    if (lane == 0)
        row_exp[m] = p;
}

// Signed byte i of a dword as f32.
__device__ __forceinline__ float code_f32(uint32_t x, int i)
{
    return (float)(int8_t)(x >> (8 * i));
}

template <class F>
__device__ __forceinline__ void split_q8_block(const uint8_t *__restrict__ aq, int p,
                                               u32x4 *__restrict__ ahl, int M, int nblk,
                                               long long R, int kb, int lane)
{
    const int li = lane & 15, g = lane >> 4;
    const long long m = R * 16 + li;
    f16x8 hi = {}, lo = {};
    if (m < M) {
        const uint8_t *blk = aq + ((size_t)m * (size_t)nblk + (size_t)kb) * kQ8Bytes;
        const float d = f16_bits_to_f32(load_u16(blk));
        // Slots 4..7 meet weights decoded at 2^kHiLog2 x their code (as in
        // split_store): they carry a further 2^-kHiLog2.
        const float sl = ldexpf(d, p), sh = ldexpf(d, p - F::kHiLog2);
        const uint32_t cl = load_u32_unaligned(blk + 2 + F::a_lo(g));
        const uint32_t ch = load_u32_unaligned(blk + 2 + F::a_hi(g));
        const float e[8] = {code_f32(cl, 0) * sl, code_f32(cl, 2) * sl, code_f32(cl, 1) * sl,
                            code_f32(cl, 3) * sl, code_f32(ch, 0) * sh, code_f32(ch, 2) * sh,
                            code_f32(ch, 1) * sh, code_f32(ch, 3) * sh};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const f16 h = (f16)e[s];
            hi[s] = h;
            lo[s] = (f16)((e[s] - (float)h) * 2048.0f);
        }
    }
    const long long mt = R >> 3;
    const long long idx = (mt * nblk + kb) * kOpsPerBlockTile + (R & 7) * 64 + lane;
    ahl[idx] = bitcast<u32x4>(hi);
    ahl[idx + 8 * 64] = bitcast<u32x4>(lo);
}

// The split path's preparation in one launch, arranged as k_gemm_prep_f32:
// workgroup (R, q) finds group R's row exponents from the whole rows' block
// scales (one row per wavefront; part 0 writes row_exp), then its wavefronts
// split the blocks of K part q in turn.
template <class F>
__global__ __launch_bounds__(64 * kPrepWaves) void k_gemm_prep_q8a(const uint8_t *__restrict__ aq,
                                                                 int *__restrict__ row_exp,
                                                                 u32x4 *__restrict__ ahl, int M,
                                                                 int K, int part_blocks)
{
    __shared__ int s_p[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long R = blockIdx.x;
    const int nblk = K >> 5;
    const int kb0 = (int)blockIdx.y * part_blocks, kb1 = min(kb0 + part_blocks, nblk);
    static_assert(kPrepWaves == 16, "one row of the group per wavefront");
    const long long m = R * 16 + wave;
    int pw = 0;
    if (R * 16 < M)
        pw = row_exp_q8a(aq + (size_t)min(m, (long long)M - 1) * (size_t)nblk * kQ8Bytes, nblk, lane);
    if (lane == 0) {
        s_p[wave] = pw;
        if (blockIdx.y == 0 && m < M)
            row_exp[m] = pw;
    }
    __syncthreads();
    const int p = s_p[lane & 15];
    for (int kb = kb0 + wave; kb < kb1; kb += kPrepWaves)
        split_q8_block<F>(aq, p, ahl, M, nblk, R, kb, lane);
}

__global__ __launch_bounds__(256) void k_q8a_to_f32(const uint8_t *__restrict__ aq,
                                                   const int *__restrict__ row_exp,
                                                   float4 *__restrict__ out, int K,
                                                   long long n_quads)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_quads)
        return;
    const long long e = i * 4;                    // K % 32 == 0: a quad never straddles blocks
    const long long m = e / K;
    const int k = (int)(e - m * K);
    const uint8_t *blk = aq + ((size_t)m * (size_t)(K >> 5) + (size_t)(k >> 5)) * kQ8Bytes;
    const float s = ldexpf(f16_bits_to_f32(load_u16(blk)), row_exp[m]);
    const uint32_t c = load_u32_unaligned(blk + 2 + (k & 31));
    out[i] = make_float4(code_f32(c, 0) * s, code_f32(c, 1) * s, code_f32(c, 2) * s,
                         code_f32(c, 3) * s);
}

template <class F>
static hipError_t launch_gemm_q8a_f(const uint8_t *aq, const uint8_t *w, float *y, int M, int N,
                                    int K, void *workspace, hipStream_t s)
{
    const int tiles_m = (M + kGemmBM - 1) / kGemmBM, tiles_n = (N + kGemmBN - 1) / kGemmBN;
    const long long T = (long long)tiles_m * tiles_n;
    if (T > 0x7fffffffLL)
        return hipErrorInvalidValue;
    int *row_exp = static_cast<int *>(workspace);
    void *act = static_cast<char *>(workspace) + q4v::gemm_row_exp_bytes(M);
    hipError_t e;
    if (!q4v::gemm_splits_activations(K) || (long long)M * N >= (1LL << 31)) {
        e = launch_kernel(k_row_exp_q8a, dim3((unsigned)((M + kRowExpWaves - 1) / kRowExpWaves)),
                          dim3(64 * kRowExpWaves), 0, s, aq, row_exp, M, K);
        if (e != hipSuccess)
            return e;
        const long long n_quads = (long long)M * K / 4;
        const long long grid = (n_quads + 255) / 256;
        if (grid > 0x7fffffffLL)
            return hipErrorInvalidValue;
        e = launch_kernel(k_q8a_to_f32, dim3((unsigned)grid), dim3(256), 0, s, aq,
                          (const int *)row_exp, static_cast<float4 *>(act), K, n_quads);
        if (e != hipSuccess)
            return e;
        return launch_any_segments<F>((const float *)act, w, y, M, N, K, tiles_m, tiles_n,
                                      row_exp, 0, s);
    }
    const long long groups = (long long)tiles_m * 8;
    const int nblk = K / 32;
    const int part_blocks = prep_part_blocks(groups, nblk, 1);
    if (groups > 0x7fffffffLL)
        return hipErrorInvalidValue;
    e = launch_kernel(k_gemm_prep_q8a<F>,
                      dim3((unsigned)groups, (unsigned)((nblk + part_blocks - 1) / part_blocks)),
                      dim3(64 * kPrepWaves), 0, s, aq, row_exp, static_cast<u32x4 *>(act), M, K,
                      part_blocks);
    if (e != hipSuccess)
        return e;
    return launch_split_segments<F, false>((const u32x4 *)act, w, y, M, N, K, tiles_m, tiles_n,
                                           row_exp, s);
}

hipError_t launch_gemm_q8a(WeightFormat fmt, const uint8_t *a_q, const uint8_t *w, float *y, int M,
                           int N, int K, void *workspace, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemm_q8a_f<FmtQ8_0>(a_q, w, y, M, N, K, workspace, s);
    return launch_gemm_q8a_f<FmtQ4_0>(a_q, w, y, M, N, K, workspace, s);
}

}  // namespace q4k
