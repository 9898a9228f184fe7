// Decode-shaped block-quantized x f32 product, y[m, n] = sum_k a[m, k] w[n, k]
// for 1 <= M <= 8 activation rows, on gfx950 matrix cores, for Q4_0 and Q8_0
// weight streams.
//
// Operation: docs.rs fuel-dispatch, "quantized (GGML) kernel contracts",
// section qmatvec_q4_0 (one row there; up to eight rows here), with the blocks
// of sections dequant_q4_0 and dequant_q8_0 (the quantized-matmul binding
// described there picks either by quant type). The work is bound by streaming
// the weight blocks once (N K 18/32 or 34/32 bytes).
//
// Design
// ------
// * One workgroup of 8 wavefronts owns 16 output columns (16 weight rows) and
//   the whole K. Wavefront w owns a contiguous run of the K/32 blocks. Lane
//   (j = lane % 16, g = lane / 16) takes, per block of weight row n0 + j, the
//   binary16 scale and the quant bytes of lane group g (formats.h): every
//   weight byte is read once, and all of a wavefront's loads are issued before
//   the activations are prepared, so HBM latency overlaps that work.
// * The 32-element dot products of a block run on v_mfma_f32_16x16x32_f16.
//   Operand B (32 x 16) holds the exact binary16 weight codes of 16 weight rows;
//   operand A (16 x 32) holds the activations split into two binary16 terms,
//   hi = f16(v) and lo = f16(v - hi) (rows 2m and 2m+1 for activation row m),
//   which together carry 22 significant bits. Each product of a binary16 pair
//   is exact and the matrix core accumulates in f32.
// * Decode (formats.h): Q4_0 nibbles become f16 pairs with one AND-OR against
//   the exponent pattern of 1024 and one packed f16 subtraction each; the high
//   nibbles are decoded in place, which yields 16 (q - 8), so the activations
//   paired with low nibbles carry the factor 16 instead and one power of two
//   restores every product. Q8_0 bytes go through one byte permute per pair and
//   the same subtraction. The K order inside a block is permuted; A uses the
//   same permutation, so the sum is unchanged.
// * Each block's f32 partial is scaled by its d into f32 accumulators
//   (d * C + acc), giving the two-level order block partial -> scale -> sum of
//   blocks. Wavefront partials are summed in LDS in a fixed order, so repeated
//   calls return identical bits.
// * Range: activation row m is scaled by a power of two 2^p_m chosen from its
//   max |a| so that the largest A value lies in [2^14, 2^15): no binary16
//   overflow, and elements far below the row maximum lose at most 2^-25 of
//   2^p_m absolutely. The scale is undone exactly on the f32 result.
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "formats.h"
#include "launch.h"
#include "validate.h"

namespace q4k {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvStreamWaves = 8;

// Split v into binary16 hi + lo with hi = f16(v) and lo = f16(v - hi).
__device__ __forceinline__ void split2(float v, f16 &hi, f16 &lo)
{
    hi = (f16)v;
    lo = (f16)(v - (float)hi);
}

// split2 of x0 sc and x1 sc (sc a power of two, so x sc is exact), packed:
// hi = (f16(x0 sc), f16(x1 sc)) and lo = (f16(x0 sc - hi0), f16(x1 sc - hi1)).
// Each half is one mixed-precision FMA (f32 operands, f16 result, one
// rounding), and lo reads its hi half straight from the packed register.
__device__ __forceinline__ void split2_pair(float x0, float x1, float sc, uint32_t &hi,
                                            uint32_t &lo)
{
    uint32_t h, l;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(h) : "v"(x0), "v"(sc));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0" : "+v"(h) : "v"(x1), "v"(sc));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,0,1]" : "=v"(l) : "v"(x0), "v"(sc), "v"(h));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "+v"(l) : "v"(x1), "v"(sc), "v"(h));
    hi = h;
    lo = l;
}

// max(m, |a|, |b|) for m >= 0, one instruction: the absolute values are
// operand modifiers, and in inline asm the compiler adds no canonicalizing
// of the loaded values (as it would for fmaxf). For finite values the result
// equals the largest cleared-sign bit pattern; only loaded activations and
// the running maximum are read (no result of an in-flight MFMA).
__device__ __forceinline__ float max3_abs(float m, float a, float b)
{
    float r;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}

// Largest A value of a row is 2^kHiLog2 max|a| 2^p: p puts it in [2^14, 2^15).
template <class F>
__device__ __forceinline__ int row_scale_exp(float am)
{
    int e = 0;
    frexpf(am, &e);                                  // am in [2^(e-1), 2^e)
    const int p = (am == 0.0f) ? 0 : 15 - F::kHiLog2 - e;
    return p > 120 ? 120 : (p < -120 ? -120 : p);
}

// bfloat16 activations (BF): a bfloat16 value has an 8-bit significand, so
// after a power-of-two scale that puts the largest A value of its row in
// [2^15, 2^16) every element within 2^28 (Q4_0) or 2^32 (Q8_0) of the row's
// largest magnitude is exactly a binary16 number. One A row per activation
// row then replaces the hi / lo pair: A row m is activation row m, and lane
// (j, g) accumulates C rows 4g..4g+3, activation rows 4g + r.
template <class F>
__device__ __forceinline__ int row_scale_exp_bf16(float am)
{
    int e = 0;
    frexpf(am, &e);                                  // am in [2^(e-1), 2^e)
    return (am == 0.0f || !(am <= 3.4e38f)) ? 0 : 16 - F::kHiLog2 - e;
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

template <bool BF, int M>
struct GemvRows {
    static constexpr int NI = BF ? M : 2 * M;                              // A rows in use
    static constexpr int NACC = BF ? (M < 4 ? M : 4) : (M == 1 ? 2 : 4);   // C rows a lane owns
    static constexpr int NOUT = BF ? NACC : NACC / 2;                      // activation rows a lane owns
    // Activation row of a lane's output h (lane group g).
    static __device__ __forceinline__ int row(int g, int h) { return BF ? 4 * g + h : 2 * g + h; }
};

template <class F, int M, bool BF>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(const void *__restrict__ a_,
                                                      const uint8_t *__restrict__ w,
                                                      float *__restrict__ y, int N, int K)
{
    constexpr int NW = kGemvWaves;
    constexpr int CB = (M <= 4) ? 128 : 64;   // blocks per K chunk held in LDS
    constexpr int PB = CB / NW;               // blocks per wavefront per chunk
    using R = GemvRows<BF, M>;
    constexpr int NI = R::NI;                 // A rows in use (hi, lo per row; hi only for BF)
    constexpr int NACC = R::NACC;             // accumulator rows a lane can own
    const float *a = static_cast<const float *>(a_);
    const uint16_t *ab = static_cast<const uint16_t *>(a_);

    __shared__ uint4 s_a[CB * 4 * NI];        // [block][g][i] 8-half A operands
    __shared__ float s_part[NW][M][16];
    __shared__ float s_amax[NW][M];
    __shared__ int s_exp[M];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nblk = K >> 5;
    const size_t row_bytes = (size_t)nblk * F::kBytes;
    const uint8_t *wrow = w + (size_t)min(n0 + j, N - 1) * row_bytes;

    uint32_t wx[PB][F::kQsDwords], wd[PB];
    auto issue_loads = [&](int cb0, int cnt) {
        const int per = (cnt + NW - 1) / NW, b0 = wave * per;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int b = b0 + u;
            if (u < per && b < cnt) {
                const uint8_t *bp = wrow + (size_t)(cb0 + b) * F::kBytes;
                wd[u] = load_u16(bp);
                load_qs<F>(bp, g, wx[u]);
            }
        }
    };
    issue_loads(0, min(CB, nblk));

    // Per-row power-of-two scale from max |a| over the whole row.
    float mx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        mx[m] = 0.0f;
        if constexpr (BF) {
            // K % 32 == 0: 8-byte groups of four bfloat16 values.
            const uint2 *row = reinterpret_cast<const uint2 *>(ab + (size_t)m * K);
            for (int f = tid; f < (K >> 2); f += kGemvThreads) {
                const uint2 v = row[f];
                mx[m] = fmaxf(mx[m], fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                                           fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))));
            }
        } else {
            const float4 *row = reinterpret_cast<const float4 *>(a + (size_t)m * K);
            for (int f = tid; f < (K >> 2); f += kGemvThreads) {
                float4 v = row[f];
                mx[m] = fmaxf(mx[m], fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            mx[m] = fmaxf(mx[m], __shfl_xor(mx[m], o));
        if (lane == 0)
            s_amax[wave][m] = mx[m];
    }
    __syncthreads();
    if (tid < M) {
        float am = 0.0f;
        for (int ww = 0; ww < NW; ++ww)
            am = fmaxf(am, s_amax[ww][tid]);
        s_exp[tid] = BF ? row_scale_exp_bf16<F>(am) : row_scale_exp<F>(am);
    }
    __syncthreads();
    int pexp[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        pexp[m] = s_exp[m];

    float acc[NACC];
#pragma unroll
    for (int r = 0; r < NACC; ++r)
        acc[r] = 0.0f;

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int nchunks = (nblk + CB - 1) / CB;
    for (int c = 0; c < nchunks; ++c) {
        const int cb0 = c * CB, cnt = min(CB, nblk - cb0);
        if (c > 0) {
            __syncthreads();                   // every wavefront is done with s_a
            issue_loads(cb0, cnt);
        }
        // A operands of this chunk: entry (b, gg, 2m) = hi, (b, gg, 2m+1) = lo,
        // slots = 2^kHiLog2 a[lo(gg) + {0,2,1,3}] then a[hi(gg) + {0,2,1,3}],
        // all x 2^p.
        for (int q = tid; q < cnt * 4 * M; q += kGemvThreads) {
            const int m = q % M, rest = q / M, gg = rest & 3, b = rest >> 2;
            if constexpr (BF) {
                // Slots as below, one binary16 term each (exact, see above).
                const uint16_t *blk = ab + (size_t)m * K + (size_t)(cb0 + b) * 32;
                const uint2 L = *reinterpret_cast<const uint2 *>(blk + F::a_lo(gg));
                const uint2 H = *reinterpret_cast<const uint2 *>(blk + F::a_hi(gg));
                const int pl = pexp[m] + F::kHiLog2, ph = pexp[m];
                const float v[8] = {ldexpf(bf16_lo(L.x), pl), ldexpf(bf16_lo(L.y), pl),
                                    ldexpf(bf16_hi(L.x), pl), ldexpf(bf16_hi(L.y), pl),
                                    ldexpf(bf16_lo(H.x), ph), ldexpf(bf16_lo(H.y), ph),
                                    ldexpf(bf16_hi(H.x), ph), ldexpf(bf16_hi(H.y), ph)};
                f16x8 hi;
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    hi[s] = (f16)v[s];
                s_a[(b * 4 + gg) * NI + m] = bitcast<uint4>(hi);
                continue;
            }
            const float *blk = a + (size_t)m * K + (size_t)(cb0 + b) * 32;
            const float4 L = *reinterpret_cast<const float4 *>(blk + F::a_lo(gg));
            const float4 H = *reinterpret_cast<const float4 *>(blk + F::a_hi(gg));
            const float sh = ldexpf(1.0f, pexp[m]), sl = (float)(1 << F::kHiLog2) * sh;
            const float v[8] = {L.x * sl, L.z * sl, L.y * sl, L.w * sl,
                                H.x * sh, H.z * sh, H.y * sh, H.w * sh};
            f16x8 hi, lo;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                f16 h, l;
                split2(v[s], h, l);
                hi[s] = h;
                lo[s] = l;
            }
            uint4 *dst = &s_a[(b * 4 + gg) * NI + 2 * m];
            dst[0] = bitcast<uint4>(hi);
            dst[1] = bitcast<uint4>(lo);
        }
        __syncthreads();

        const int per = (cnt + NW - 1) / NW, b0 = wave * per;
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const int b = b0 + u;
            if (u < per && b < cnt) {          // uniform across the wavefront
                f16x8 aop = {};
                if (j < NI)
                    aop = bitcast<f16x8>(s_a[(b * 4 + g) * NI + j]);
                const f16x8 bop = F::decode(wx[u], F::kMagic);
                const f32x4 C = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, zero4, 0, 0, 0);
                const float d = f16_bits_to_f32(wd[u]);
#pragma unroll
                for (int r = 0; r < NACC; ++r)
                    acc[r] = fmaf(d, C[r], acc[r]);
            }
        }
    }

    // Lane (j, g) holds C rows 4g..4g+3 of column j: activation rows 2g (hi, lo)
    // and 2g+1 (hi, lo), or for BF activation rows 4g..4g+3.
#pragma unroll
    for (int h = 0; h < R::NOUT; ++h) {
        const int m = R::row(g, h);
        if (m < M)
            s_part[wave][m][j] = BF ? acc[h] : acc[2 * h] + acc[2 * h + 1];
    }
    __syncthreads();
    if (tid < M * 16) {
        const int m = tid >> 4, jj = tid & 15, n = n0 + jj;
        float s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            s += s_part[ww][m][jj];
        if (n < N)
            y[(size_t)m * N + n] = ldexpf(s, -pexp[m] - F::kHiLog2);
    }
}

// ---------------------------------------------------------------------------
// Streaming variant for rows that are 16-byte aligned (K % 256 == 0), which
// covers the decode shapes. Same arithmetic as above; what changes is how the
// weight bytes reach the matrix cores:
// * Each wavefront owns a run of blocks of the workgroup's 16 rows and walks it
//   in chunks of CH blocks (CH * 18 or CH * 34 bytes per row, a multiple of
//   16 for CH = 8 or 16). A chunk is fetched with aligned 16-byte loads, lane (r, c) taking
//   16-byte column c of row r, and written unchanged into the wavefront's own
//   LDS area. Operands are then read back with aligned LDS dword pairs and
//   realigned with v_alignbyte. No global load is narrower than 16 bytes or
//   misaligned, and the next chunk's loads are in flight while the current
//   one is computed.
// * The activations of a chunk are split by the whole wavefront (each lane a
//   few 8-element groups) and passed to the A-operand lanes through LDS. The
//   power-of-two scale is chosen per (chunk, activation row) from the chunk's
//   own max |a|, and undone on that chunk's f32 partial, so no workgroup-wide
//   pass over the activations is needed.
// * Wavefront partials meet in LDS once, at the end, and are summed in a
//   fixed order.

// Order LDS traffic between the lanes of one wavefront: its LDS operations
// execute in issue order, so it is enough that the compiler keeps them there.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <class F, int M, int NW, int CH_, bool BF, int RPW_ = 16, bool LA_ = false>
struct GemvStreamCfg {
    static constexpr int CH = CH_;                        // blocks per chunk (8 or 16)
    static constexpr int RPW = RPW_;                      // weight rows per workgroup (16 or 8)
    // LA (line-aligned loads; rows a whole number of 128-byte lines from a
    // line-aligned base): a chunk row is fetched as the NLN whole lines that
    // hold it. A chunk starts at a multiple of its byte count, so its offset
    // into its first line is a multiple of that count's lowest set bit, at
    // most kMaxShift; from every such offset it spans exactly NLN lines
    // (asserted), so the lines never pass the end of the row.
    static constexpr bool LA = LA_;
    static constexpr int kChunkBytes = CH * F::kBytes;
    static constexpr int kMaxShift = (kChunkBytes & 127) == 0 ? 0 : 128 - (kChunkBytes & -kChunkBytes);
    static constexpr int NLN = (kMaxShift + kChunkBytes + 127) / 128;
    static_assert(!LA || (kChunkBytes + 127) / 128 == NLN,
                  "a chunk spans the same number of lines from every start offset");
    static constexpr int CPR = LA ? 8 * NLN : CH * F::kBytes / 16;   // 16-byte columns per staged row
    // Weight loads: eight lanes per row take 128 contiguous bytes (one cache
    // line's worth), eight rows per load: loads (RPW / 8) c + h cover columns
    // 8c..8c+7 of rows 8h..8h+7, for each of the NG whole groups of eight
    // columns; one more load covers the TC tail columns of all RPW rows
    // (TLPR = 64 / RPW lanes per row).
    static constexpr int NG = CPR / 8, TC = CPR % 8, RH = RPW / 8, TLPR = 64 / RPW;
    static constexpr int NLOAD = RH * NG + (TC > 0 ? 1 : 0);   // 16-byte loads per lane per chunk
    static constexpr int RS = 16 * CPR + 16;              // LDS bytes per staged row
    static constexpr int WBYTES = RPW * RS;               // staged weight bytes per wavefront
    static constexpr int NI = GemvRows<BF, M>::NI;        // A rows in use
    // The A operands of a chunk pass through LDS in AH halves when a whole
    // chunk's would not fit (16 blocks of more than eight A rows).
    static constexpr int AH = (CH == 16 && NI > 8) ? 2 : 1;
    static constexpr int CHH = CH / AH;                   // blocks per A pass
    static constexpr int ABYTES = CHH * 4 * NI * 16;      // A operands per wavefront
    // Activation split: lane l handles activation row l / QN (QN = 64 / MP,
    // MP = M rounded up to a power of two) and, in each A pass, the 8-element
    // groups l % QN + QN r (r < EPP) of that pass's 4 CHH (block, lane group)
    // pairs, so consecutive lanes read consecutive activations.
    static constexpr int MP = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8));
    static constexpr int QN = 64 / MP;                    // lanes per activation row
    static constexpr int EPP = (4 * CHH + QN - 1) / QN;   // groups per lane per A pass
    static constexpr int EPL = AH * EPP;                  // ... per chunk
    static constexpr int LDS_PER_WAVE = WBYTES + ABYTES;
    static constexpr int NPART = CH == 16 ? 4 : 2;        // parts a chunk is contracted in
    // Loads (per lane) that hold every byte of the chunk's first b blocks.
    static constexpr int cols_for(int b) { return (F::kBytes * b + 15) / 16; }
    // LA: the lines that hold them at the largest start offset.
    static constexpr int loads_for(int b)
    {
        if constexpr (LA)
            return b == 0 ? 0 : RH * min_c((kMaxShift + F::kBytes * b + 127) / 128, NLN);
        return b == 0 ? 0 : (cols_for(b) <= 8 * NG ? RH * ((cols_for(b) + 7) / 8) : NLOAD);
    }
    static constexpr int min_c(int x, int y) { return x < y ? x : y; }
    static_assert(RPW == 8 || RPW == 16, "eight or sixteen weight rows per workgroup");
    static_assert(TC <= TLPR, "the tail columns fit the lanes of a row");
    static_assert(CH == 8 || CH == 16, "chunks are 8 or 16 blocks");
    static_assert((CH * F::kBytes) % 16 == 0, "a chunk row is whole 16-byte columns");
};

// Calls f(integral_constant<int, P>) for P = 0 .. NP-1, in order.
template <int NP, class F, int... P>
__device__ __forceinline__ void for_each_part_impl(F &&f, std::integer_sequence<int, P...>)
{
    (f(std::integral_constant<int, P>{}), ...);
}
template <int NP, class F>
__device__ __forceinline__ void for_each_part(F &&f)
{
    for_each_part_impl<NP>(f, std::make_integer_sequence<int, NP>{});
}

// Maximum of a non-negative float over the wavefront, returned to every lane.
// Non-negative IEEE floats order like their bit patterns, so the reduction
// runs on integers: DPP within quads, half-rows and rows, then one readlane
// per row of 16 lanes.
__device__ __forceinline__ float wave_max_nonneg(float v)
{
    int x = __builtin_bit_cast(int, v);
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));   // row_half_mirror
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));   // row_mirror
    const int r = max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
                      max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
    return __builtin_bit_cast(float, r);
}

// Maximum of a non-negative float over each run of QN consecutive lanes (QN
// = 8, 16, 32 or 64), returned to each lane of the run: DPP within quads,
// half-rows and rows, then across rows.
template <int QN>
__device__ __forceinline__ float lane_run_max_nonneg(float v)
{
    static_assert(QN == 8 || QN == 16 || QN == 32 || QN == 64, "runs of 8, 16, 32 or 64 lanes");
    if constexpr (QN == 64) {
        return wave_max_nonneg(v);
    } else {
        int x = __builtin_bit_cast(int, v);
        x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
        x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
        x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));   // row_half_mirror
        if constexpr (QN >= 16)
            x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));   // row_mirror
        if constexpr (QN >= 32)
            x = max(x, __shfl_xor(x, 16));
        return __builtin_bit_cast(float, x);
    }
}

// A operand (block b, lane group g, A row i) sits in LDS at slot
// b ASTRIDE / 16 + g NI + (i ^ a_swz<NI>(b, g)). A write instruction of the
// activation split has eight consecutive lanes on one A row (or hi / lo
// pair) of two consecutive blocks times the four lane groups; unswizzled,
// NI a multiple of 8 puts all eight in one bank group. The XOR, below NI,
// gives each of the eight its own 16-byte bank group, and within one (b, g)
// it only permutes the NI slots, so the operand reads (lane j of group g
// reads row j) stay conflict-free. Other NI keep the plain layout, where the
// conflicts are at most four-way.
template <int NI>
__device__ __forceinline__ int a_swz(int b, int g)
{
    if constexpr (NI == 8 || NI == 16)
        return ((b & 1) << 2) | g;
    else if constexpr (NI == 4)
        return ((b & 1) << 1) | (g >> 1);
    else if constexpr (NI == 2)
        return b & 1;
    else
        return 0;
}

// Calls f(integral_constant<int, B>) for B = B0 .. B1-1, in order.
template <int B0, class F, int... P>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, P...>)
{
    (f(std::integral_constant<int, B0 + P>{}), ...);
}
template <int B0, int B1, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl<B0>(f, std::make_integer_sequence<int, B1 - B0>{});
}

// NT: the weight loads are non-temporal. With whole-line loads (LA, below) on
// every launch. Otherwise where every wavefront streams one chunk and no
// second workgroup shares its compute unit (about 6% faster at 1 x 4096 x
// 4096 and 8 x 4096 x 4096), and by the row-group loops (LN) from two
// activation rows; with partial lines and more chunks per wavefront or
// workgroups per compute unit it was 3-5% slower.
// MODE 0: as above. MODE 1 (AL): the MFMAs read the chunk's A operands from
// LDS block by block instead of holding all of them in registers (only where
// one pass holds the chunk's A operands, AH == 1). That frees CH * 4 VGPRs, so
// two workgroups share a compute unit and one's loads overlap the other's
// work: taken when there are more workgroups than compute units (and LN,
// below, does not apply) or more than one chunk per wavefront. MODE 2 (PA, f32 activations): `a` holds operands
// prepared once by k_gemv_prep_ops (the two-term A operands of every block in
// [block][lane group][A row] order, then the per-row exponents), loaded
// straight into the A registers: no per-chunk split, scale or LDS pass.
// LN (MODE 0 or 2, one chunk per wavefront, no K split): the workgroup
// walks the row groups blockIdx.x, blockIdx.x + gridDim.x, ... of 16 weight
// rows with the same chunk, so its activations are loaded and split (or its
// prepared operands loaded) once for all of them; once a group's weight bytes
// are staged, the next group's loads are issued, and each group ends with its
// own reduction and store (partials in alternate LDS buffers, one barrier per
// group). Every output sees the same arithmetic as without LN.
// LA (weight rows a whole number of 128-byte lines from a line-aligned base):
// each chunk row is fetched as the whole lines that hold it, starting at the
// line of its first byte, so no load instruction touches part of a line (up to
// a line more per row than the chunk's bytes; the lines a neighbouring
// wavefront also fetches are cache hits). The staged chunk row then begins
// (chunk byte offset mod 128) bytes into the staged lines. Same arithmetic.
template <class F, int M, int NW, int CH, bool BF, int MODE, int RPW = 16, bool NT = false,
          bool LN = false, bool LA = false>
__global__ __launch_bounds__(64 * NW) void k_gemv_stream(const void *__restrict__ a,
                                                        const uint8_t *__restrict__ w,
                                                        float *__restrict__ y, int N, int K,
                                                        int ks)
{
    using C = GemvStreamCfg<F, M, NW, CH, BF, RPW, LA>;
    using R = GemvRows<BF, M>;
    constexpr bool AL = MODE == 1, PA = MODE == 2;
    static_assert(!AL || C::AH == 1, "A operands read from LDS need the whole chunk's in one pass");
    static_assert(!PA || !BF, "prepared operands are made from f32 activations");
    static_assert(!LN || MODE != 1, "row-group loops keep the A operands in registers");
    constexpr int NACC = R::NACC;
    constexpr uint32_t ES = BF ? 2 : 4;           // bytes per activation
    constexpr int ASTRIDE = 4 * C::NI * 16;       // A bytes per block

    // Per wavefront: [staged weight bytes | A operands].
    // PA needs no A area: its operands go straight to registers.
    constexpr int kLdsPerWave = PA ? C::WBYTES : C::LDS_PER_WAVE;
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[NW * kLdsPerWave];
    __shared__ float s_part[LN ? 2 : 1][NW][M][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    int n0 = blockIdx.x * RPW;
    const int nblk = K >> 5;
    const uint32_t row_bytes = (uint32_t)nblk * F::kBytes;
    uint8_t *s_w = s_mem + wave * kLdsPerWave;
    uint8_t *s_a = s_w + C::WBYTES;

    // The workgroup's K split: blocks [kb_lo, kb_hi) (the whole row unless the
    // call splits K across workgroups, blockIdx.y being the split; each split
    // then writes its own partial y, M x N f32, at y + split M N), a whole
    // number of CH-block chunks (the host picks CH so). The chunks are dealt
    // to the wavefronts in turn: wavefront w takes chunks w, w + NW, ... So
    // the chunk size depends only on K, not on how K divides among the
    // wavefronts, and long rows keep 16-block chunks (more bytes in flight).
    const int kb_lo = (int)blockIdx.y * ks, kb_hi = min(kb_lo + ks, nblk);
    const int wb0 = kb_lo + wave * C::CH;       // this wavefront's first chunk
    constexpr int kStride = NW * C::CH;         // ... and the step to its next
    y += (size_t)blockIdx.y * (size_t)M * (size_t)N;

    // Loader role (GemvStreamCfg): in load i < RH NG, row lrow + 8 (i % RH),
    // column lcol + 8 (i / RH); in the tail load, row trow, column
    // 8 NG + tcol (clamped to the last column: surplus lanes re-read it).
    // Each load thus touches one cache line's worth per row, eight rows.
    const int lrow = lane >> 3, lcol = lane & 7, trow = lane / C::TLPR, tcol = lane % C::TLPR;
    uint32_t row_off0, row_off1, tail_off;
    auto set_rows = [&](int r0) __attribute__((always_inline)) {
        row_off0 = (uint32_t)min(r0 + lrow, N - 1) * row_bytes;
        row_off1 = (uint32_t)min(r0 + lrow + 8, N - 1) * row_bytes;
        tail_off = (uint32_t)min(r0 + trow, N - 1) * row_bytes +
                   16u * (uint32_t)(8 * C::NG + min(tcol, C::TC > 0 ? C::TC - 1 : 0));
    };
    set_rows(n0);

    u32x4 wreg[C::NLOAD];
    // Four activations per half group: f32, or bfloat16 pairs.
    using AV = std::conditional_t<BF, uint2, float4>;
    AV areg[C::EPL][2];
    // Entry r of a lane: A pass h = r / EPP, group c = sq + QN (r % EPP) of
    // that pass (block h CHH + c / 4 of the chunk, lane group gg = c % 4), row
    // sm: elements lo(gg)..lo(gg)+3 and hi(gg)..hi(gg)+3. Activations are
    // requested first (vmcnt drains in issue order), so their split overlaps
    // the weight loads.
    const int sq = lane % C::QN, sm = lane / C::QN;
    const int sm_ld = min(sm, M - 1);
    const uint8_t *a8 = reinterpret_cast<const uint8_t *>(a);
    // Every lane issues every load (surplus lanes re-read an in-bounds group or
    // column that is then ignored), so the compiler's in-order wait counts are
    // exact and the first half of a chunk waits only for its own loads.
    auto fetch_impl = [&](int cb0, auto acts_c) __attribute__((always_inline)) {
        constexpr bool kActs = decltype(acts_c)::value && !PA;
#pragma unroll
        for (int r = 0; r < (kActs ? C::EPL : 0); ++r) {
            const int c = min(sq + C::QN * (r % C::EPP), 4 * C::CHH - 1);
            const int b = (r / C::EPP) * C::CHH + (c >> 2), gg = c & 3;
            const uint32_t off = ((uint32_t)sm_ld * K + (uint32_t)(cb0 + b) * 32 + F::a_lo(1) * gg) * ES;
            areg[r][0] = *reinterpret_cast<const AV *>(a8 + off);
            areg[r][1] = *reinterpret_cast<const AV *>(a8 + off + ES * (F::a_hi(0) - F::a_lo(0)));
        }
        // The scheduling barriers keep the loads in column order. LA: the
        // columns count from the line that holds the chunk's first byte.
        const uint32_t cbo = ((uint32_t)cb0 * F::kBytes) & (LA ? ~127u : ~0u);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < C::RH * C::NG; ++i) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                w + ((i % C::RH ? row_off1 : row_off0) + cbo + 16u * (uint32_t)(lcol + 8 * (i / C::RH))));
            wreg[i] = NT ? __builtin_nontemporal_load(src) : *src;
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (C::TC > 0)
        {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(w + (tail_off + cbo));
            wreg[C::RH * C::NG] = NT ? __builtin_nontemporal_load(src) : *src;
        }
        // Issue point: the weight pointer escapes into an empty asm statement
        // with a memory clobber, so no pass sinks the loads below this line,
        // and the scheduling barrier keeps later work (which waits on loads)
        // from being hoisted above them.
        asm volatile("" ::"s"(w) : "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto fetch = [&](int cb0) __attribute__((always_inline)) { fetch_impl(cb0, std::true_type{}); };
    auto fetch_w = [&](int cb0) __attribute__((always_inline)) { fetch_impl(cb0, std::false_type{}); };

    // Unconditional, so no copies of the loaded registers are needed after a
    // branch (they would wait for the loads). A wavefront without blocks
    // (possible only when the workgroup's share is short) fetches the last full
    // chunk of the row, K/32 >= CH, and never reads it.
    // A operands of a chunk live in registers (set by split_activations, or
    // for PA loaded by fetch_ops).
    f16x8 aop[C::CH];
    // PA: the chunk's prepared operands, operand (b, g, i) of block cb0 + b at
    // ((cb0 + b) * 4 + g) * NI + i. Only lanes j < NI load: the other A rows
    // belong to no activation row and only fill MFMA rows that are never read.
    const u32x4 *ops = static_cast<const u32x4 *>(a);
    auto fetch_ops = [&](int cb0) __attribute__((always_inline)) {
        if constexpr (PA) {
            if (j < C::NI) {
#pragma unroll
                for (int b = 0; b < C::CH; ++b)
                    aop[b] = bitcast<f16x8>(ops[((size_t)(cb0 + b) * 4 + g) * C::NI + j]);
            }
        }
    };
    // The first chunk: prepared operands first (their loads drain before the
    // weights', so part 0 waits only for its own weight bytes), then weights.
    fetch_ops(min(wb0, nblk - C::CH));
    fetch(min(wb0, nblk - C::CH));
    // Clamped, so the address stays inside the A area even where the read is
    // masked off.
    // Operand reads: lane (g, j) reads A row j of lane group g; the swizzle
    // depends on the block's parity (ASTRIDE is a whole number of slots).
    const int jr = min(j, C::NI - 1);
    const uint8_t *a_lane0 = s_a + (g * C::NI + (jr ^ a_swz<C::NI>(0, g))) * 16;
    const uint8_t *a_lane1 = s_a + (g * C::NI + (jr ^ a_swz<C::NI>(1, g))) * 16;
    // The decode's exponent pattern in a VGPR (one v_mov at kernel start; no
    // MFMA is in flight there).
    const uint32_t magic_v = magic_vgpr<F>();

    float ysum[R::NOUT];
#pragma unroll
    for (int h = 0; h < R::NOUT; ++h)
        ysum[h] = 0.0f;

    // Activation split of the chunk whose loads are in areg: per-row scale
    // from the chunk's own max |a|, then the two-term A operands into s_a.
    // It runs as soon as those loads land, never across a loop back edge, so
    // no copy of the loaded registers is kept alive while the weight loads are
    // being issued.
    int pexp[M];
    if constexpr (PA) {
        // The per-row exponents follow the operands.
        const int *row_exp = reinterpret_cast<const int *>(ops + (size_t)nblk * 4 * C::NI);
#pragma unroll
        for (int m = 0; m < M; ++m)
            pexp[m] = row_exp[m];
    }
    auto split_activations = [&]() __attribute__((always_inline)) {
        if constexpr (PA)
            return;
        // Every entry of a lane belongs to its row sm: one running maximum,
        // then one reduction over the lanes of the row. Clamped entries repeat
        // a group of the same row and lanes sm >= M a row that is never used,
        // so neither needs a mask here.
        // f32: |a| through v_max3_f32 with absolute-value modifiers, two
        // elements an instruction; bfloat16: the halves compared as integers
        // (non-negative floats order like their bit patterns), two at a time.
        uint32_t mb = 0;
        u16x2 mb16 = {0, 0};
        float mf = 0.0f;
        constexpr uint32_t kAbs2 = 0x7fff7fffu;
#pragma unroll
        for (int r = 0; r < C::EPL; ++r) {
            if constexpr (BF) {
                const uint2 L = areg[r][0], H = areg[r][1];
                mb16 = __builtin_elementwise_max(
                    mb16, __builtin_elementwise_max(bitcast<u16x2>(L.x & kAbs2), bitcast<u16x2>(L.y & kAbs2)));
                mb16 = __builtin_elementwise_max(
                    mb16, __builtin_elementwise_max(bitcast<u16x2>(H.x & kAbs2), bitcast<u16x2>(H.y & kAbs2)));
            } else {
                const float4 L = areg[r][0], H = areg[r][1];
                mf = max3_abs(max3_abs(mf, L.x, L.y), L.z, L.w);
                mf = max3_abs(max3_abs(mf, H.x, H.y), H.z, H.w);
            }
        }
        if constexpr (BF)
            mb = (uint32_t)max(mb16.x, mb16.y) << 16;
        else
            mb = __float_as_uint(mf);
        const float am = lane_run_max_nonneg<C::QN>(__uint_as_float(mb));
        const int pe = BF ? row_scale_exp_bf16<F>(am) : row_scale_exp<F>(am);
        // Lane m QN holds row m's exponent; the epilogue needs every row's.
#pragma unroll
        for (int m = 0; m < M; ++m)
            pexp[m] = __builtin_amdgcn_readlane(pe, m * C::QN);
        // Each pass writes the groups of its blocks and reads them back as A
        // operands at once; the next pass reuses the same LDS area. A lane's
        // groups share its lane group gg = sq % 4 and block parity (sq / 4) % 2
        // (QN / 4 is even), so its slots within a block are fixed.
        const int gg = sq & 3, sw = a_swz<C::NI>(sq >> 2, gg);
        const int slot_hi = gg * C::NI + ((BF ? sm : 2 * sm) ^ sw);
        const int slot_lo = gg * C::NI + ((2 * sm + 1) ^ sw);
#pragma unroll
        for (int h = 0; h < C::AH; ++h) {
        if (h > 0)
            wave_lds_sync();   // the previous pass's reads precede these writes
#pragma unroll
        for (int rr = 0; rr < C::EPP; ++rr) {
            const int r = h * C::EPP + rr, c = sq + C::QN * rr;
            if ((C::QN * C::EPP == 4 * C::CHH || c < 4 * C::CHH) && (C::MP == M || sm < M)) {
                uint8_t *blk = s_a + (c >> 2) * ASTRIDE;
                if constexpr (BF) {
                    const uint2 L = areg[r][0], H = areg[r][1];
                    const int pl = pe + F::kHiLog2;
                    const float v[8] = {ldexpf(bf16_lo(L.x), pl), ldexpf(bf16_lo(L.y), pl),
                                        ldexpf(bf16_hi(L.x), pl), ldexpf(bf16_hi(L.y), pl),
                                        ldexpf(bf16_lo(H.x), pe), ldexpf(bf16_lo(H.y), pe),
                                        ldexpf(bf16_hi(H.x), pe), ldexpf(bf16_hi(H.y), pe)};
                    f16x8 hi;
#pragma unroll
                    for (int s = 0; s < 8; ++s)
                        hi[s] = (f16)v[s];
                    *reinterpret_cast<u32x4 *>(blk + slot_hi * 16) = bitcast<u32x4>(hi);
                } else {
                    // sc the power of two (times 2^kHiLog2 on slots 0..3);
                    // slots (L.x, L.z, L.y, L.w, H.x, H.z, H.y, H.w).
                    const float sh = ldexpf(1.0f, pe), sl = (float)(1 << F::kHiLog2) * sh;
                    const float4 L = areg[r][0], H = areg[r][1];
                    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
                    split2_pair(L.x, L.z, sl, h0, l0);
                    split2_pair(L.y, L.w, sl, h1, l1);
                    split2_pair(H.x, H.z, sh, h2, l2);
                    split2_pair(H.y, H.w, sh, h3, l3);
                    *reinterpret_cast<u32x4 *>(blk + slot_hi * 16) = u32x4{h0, h1, h2, h3};
                    *reinterpret_cast<u32x4 *>(blk + slot_lo * 16) = u32x4{l0, l1, l2, l3};
                }
            }
        }
        // A operands into registers now, while the weight bytes are still in
        // flight. Only lanes j < NI read: the other A rows belong to no
        // activation row and only fill MFMA output rows that are never read.
        wave_lds_sync();
        if (!AL && j < C::NI) {
#pragma unroll
            for (int b = h * C::CHH; b < (h + 1) * C::CHH; ++b)
                aop[b] = *reinterpret_cast<const f16x8 *>((b & 1 ? a_lane1 : a_lane0) +
                                                          (b - h * C::CHH) * ASTRIDE);
        }
        }
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    split_activations();
    // Epilogue of one row group: wavefront partials into LDS (buffer buf),
    // then summed in wavefront order and stored.
    auto write_out = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < R::NOUT; ++h) {
            const int m = R::row(g, h);
            if (m < M && j < RPW)
                s_part[buf][wave][m][j] = ysum[h];
            ysum[h] = 0.0f;
        }
        __syncthreads();
        if (tid < M * RPW) {
            const int m = tid / RPW, jj = tid % RPW, n = n0 + jj;
            float sum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww)
                sum += s_part[buf][ww][m][jj];
            if (n < N)
                y[(size_t)m * N + n] = sum;
        }
    };
    // LN: this workgroup's row group (it walks groups blockIdx.x, + gridDim.x, ...).
    int rg = blockIdx.x, it = 0;
    for (int cb0 = wb0; cb0 < kb_hi; cb0 += LN ? 0 : kStride) {
        const bool more = LN ? (rg + (int)gridDim.x) * RPW < N : cb0 + kStride < kb_hi;
        // The chunk is contracted in NPART parts. Part p needs only loads
        // [0, loads_for(end of p)) of every lane, which drain first (vmcnt
        // counts in issue order), so its decode and MFMAs run while the rest of
        // the chunk is still arriving.
        auto stage = [&](auto i0_c, auto i1_c) __attribute__((always_inline)) {
            constexpr int I0 = decltype(i0_c)::value, I1 = decltype(i1_c)::value;
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                if (i < C::RH * C::NG)
                    *reinterpret_cast<u32x4 *>(s_w + (lrow + 8 * (i % C::RH)) * C::RS +
                                               16 * (lcol + 8 * (i / C::RH))) = wreg[i];
                else if (tcol < C::TC)
                    *reinterpret_cast<u32x4 *>(s_w + trow * C::RS + 16 * (8 * C::NG + tcol)) = wreg[i];
            }
        };
        float acc[NACC];
#pragma unroll
        for (int r = 0; r < NACC; ++r)
            acc[r] = 0.0f;
        // Block b of the staged row starts at byte kBytes b; read_qs realigns the
        // quant bytes of lane group g where they straddle dwords. All MFMAs of a
        // part are issued before its scale FMAs, so the matrix-core latency
        // overlaps the decode of the following blocks.
        // Lane j decodes weight row j; with eight rows per workgroup the
        // upper eight MFMA columns repeat row 7 and are never read.
        // LA: the chunk starts (cb0 kBytes) mod 128 bytes into the staged lines.
        const uint8_t *wl = s_w + min(j, C::RPW - 1) * C::RS +
                            (LA ? (((uint32_t)cb0 * F::kBytes) & 127u) : 0u);
        const uint32_t *wrow32 = reinterpret_cast<const uint32_t *>(wl);
        auto contract = [&](auto b0_c, auto b1_c) __attribute__((always_inline)) {
            constexpr int B0 = decltype(b0_c)::value, B1 = decltype(b1_c)::value;
            f32x4 Cv[B1 - B0];
            float d[B1 - B0];
            static_for<B0, B1>([&](auto b_c) __attribute__((always_inline)) {
                constexpr int b = decltype(b_c)::value;
                uint32_t x[F::kQsDwords];
                read_qs<F, b>(wrow32, g, x);
                d[b - B0] = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(wl + b * F::kBytes));
                f16x8 av;
                if constexpr (AL)
                    av = *reinterpret_cast<const f16x8 *>((b & 1 ? a_lane1 : a_lane0) + b * ASTRIDE);
                else
                    av = aop[b];
                Cv[b - B0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, F::decode(x, magic_v),
                                                                     zero4, 0, 0, 0);
            });
#pragma unroll
            for (int u = 0; u < B1 - B0; ++u)
#pragma unroll
                for (int r = 0; r < NACC; ++r)
                    acc[r] = fmaf(d[u], Cv[u][r], acc[r]);
            // Keep every MFMA result register allocated up to here: rows this
            // lane does not accumulate would otherwise be handed to the next
            // decode while the MFMA is still writing them (a stall on each).
#pragma unroll
            for (int u = 0; u < B1 - B0; ++u)
                asm volatile("" ::"v"(Cv[u]));
        };
        // Undo this chunk's scale (and the factor 2^kHiLog2) on its partial.
        auto finish_chunk = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < R::NOUT; ++h) {
                const int m = R::row(g, h);
                int pm = 0;
#pragma unroll
                for (int mm = 0; mm < M; ++mm)
                    if (mm == m)
                        pm = pexp[mm];
                ysum[h] += ldexpf(BF ? acc[h] : acc[2 * h] + acc[2 * h + 1], -pm - F::kHiLog2);
            }
        };
        // In the row-group loops, and where a wavefront walks several chunks
        // (the launches with the A operands in LDS or plain loads), a group's
        // or chunk's bytes have mostly landed by the time its wavefront gets
        // to them (they were requested one round earlier), so parts no longer
        // overlap arrival and only chain LDS round trips: Q4_0 takes 8-block
        // parts there (1 x 14336 x 4096 8.75 -> 8.48 us, 1 x 11008 x 2048
        // 5.19 -> 4.98, 1 x 4096 x 14336 8.51 -> 8.25, bfloat16 1 x 4096 x
        // 14336 8.37 -> 7.86; Q8_0 was 1-2% slower with fewer parts). With
        // whole-line loads a Q4_0 chunk's first and second halves wait for the
        // same loads as the parts within them, so they are one part each there
        // too (1 x 4096 x 4096 4.15 -> 4.11 us, 4 x 4096 x 4096 5.22 -> 5.12).
        constexpr bool kRounds = LN || (MODE == 1 && RPW == 16) || (MODE == 0 && !NT);
        constexpr int NPX = ((kRounds || LA) && F::kBytes == kQ4Bytes) ? CH / 8 : C::NPART;
        for_each_part<NPX>([&](auto p_c) __attribute__((always_inline)) {
            constexpr int P = decltype(p_c)::value;
            constexpr int B0 = P * C::CH / NPX, B1 = (P + 1) * C::CH / NPX;
            constexpr int L0 = C::loads_for(B0), L1 = C::loads_for(B1);
            stage(std::integral_constant<int, L0>{}, std::integral_constant<int, L1>{});
            auto run_part = [&]() __attribute__((always_inline)) {
                wave_lds_sync();
                contract(std::integral_constant<int, B0>{}, std::integral_constant<int, B1>{});
            };
            if constexpr (P < NPX - 1) {
                run_part();
            } else if (LN && more) {
                // Every load of this group is staged: prefetch the next
                // group's weights for the same chunk, then finish this one.
                set_rows((rg + (int)gridDim.x) * RPW);
                fetch_w(cb0);
                run_part();
                finish_chunk();
            } else if (more) {
                // Every load of this chunk is staged: prefetch the next chunk,
                // finish this one, then split the next chunk's activations (PA:
                // load its prepared operands, once this chunk's are used). The
                // fetch and the split sit in one branch, so the loaded
                // activation registers never meet a join.
                fetch(cb0 + kStride);
                run_part();
                finish_chunk();
                wave_lds_sync();   // this chunk's LDS reads precede the next chunk's writes
                split_activations();
                fetch_ops(cb0 + kStride);
            } else {
                run_part();
                finish_chunk();
            }
        });
        if constexpr (LN) {
            write_out(it & 1);
            if (!more)
                break;
            rg += (int)gridDim.x;
            ++it;
            n0 = rg * RPW;
            wave_lds_sync();   // this group's LDS reads precede the next group's writes
        }
    }
    if constexpr (!LN)
        write_out(0);
}

// Sums the partials of a K-split GEMV in split order: y[i] = sum_s part[s][i].
__global__ __launch_bounds__(256) void k_gemv_split_sum(const float *__restrict__ part,
                                                       float *__restrict__ y, long long n,
                                                       int splits)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float acc = part[i];
    for (int sp = 1; sp < splits; ++sp)
        acc += part[(long long)sp * n + i];
    y[i] = acc;
}


// True where every weight row is a whole number of 128-byte lines from a
// line-aligned base (K % 2048 == 0 in either format), so the streaming kernels
// can fetch whole lines (LA). Against loads that start at each chunk's first
// byte (same process, cold, bit-identical results): 1 x 4096 x 4096 4.24 ->
// 4.15 us, 2 x 4096 x 4096 4.85 -> 4.60, 1 x 4096 x 2048 3.44 -> 3.28, Q8_0
// 1 x 4096 x 4096 5.64 -> 5.31. With them the non-temporal hint pays on every
// launch (it cost 1.5-5% with partial lines where a compute unit holds two
// workgroups or a wavefront walks several chunks): 1 x 14336 x 4096 9.07 ->
// 8.69 us, 1 x 4096 x 14336 8.86 -> 8.56, 1 x 11008 x 2048 5.66 -> 5.16, Q8_0
// 1 x 4096 x 14336 13.7 -> 12.5.
template <class F>
static bool gemv_rows_line_aligned(const uint8_t *w, int K)
{
    return ((size_t)(K / 32) * F::kBytes) % 128 == 0 && ((uintptr_t)w & 127u) == 0;
}

template <class F, int M, bool BF, bool LA>
static hipError_t launch_gemv_m_la(const void *a, const uint8_t *w, float *y, int N, int K,
                                   hipStream_t s, const q4v::GemvSplit &sp)
{
    const unsigned grid = (unsigned)((N + 15) / 16);
    // Streaming path: 16-byte aligned rows (K % 256 == 0, so K/32 % 8 == 0 and
    // a row is a whole number of 16-byte columns in either format) and 32-bit
    // byte offsets. Chunks of 16 blocks when every split's length divides by
    // 16 (at K = 4096, one chunk and one memory round trip per wavefront), else 8.
    constexpr int NW = kGemvStreamWaves;
    const int nblk = K / 32;
    if (q4v::gemv_streams(M, N, K, F::kBytes, BF ? 2 : 4)) {
        // K split across sp.splits workgroups of ks blocks each (one split: ks = K/32).
        const int splits = sp.splits > 1 ? sp.splits : 1;
        const int ks = splits > 1 ? sp.ks : nblk, kl = nblk - (splits - 1) * ks;
        const dim3 g2(grid, (unsigned)splits);
        const int ch = q4v::gemv_chunk_blocks(ks, kl);
        // A operands from LDS when a compute unit gets more than one workgroup
        // or a wavefront more than one chunk (and one pass holds them);
        // otherwise, or with whole-line loads, the weight loads are
        // non-temporal (NT).
        const bool al = (long long)grid * splits > 256 || ks > NW * ch;
        // One activation row, a grid of at most half the compute units and one
        // chunk per wavefront (1x512x4096, 1x2048x4096: 5% and 4% faster):
        // eight weight rows per workgroup instead, twice the workgroups, with
        // the A operands in LDS. At 4096 rows (one workgroup per compute unit)
        // or longer K the doubled per-workgroup split and reduction cost more
        // (1x4096x4096 4.53 -> 5.23 us, 1x4096x14336 8.9 -> 11.6 us).
        if constexpr (M == 1)
            if (splits == 1 && ch == 16 && grid <= 128 && ks <= NW * ch)
                return launch_kernel(k_gemv_stream<F, 1, NW, 16, BF, 1, 8, true, false, LA>,
                                     dim3((unsigned)((N + 7) / 8), 1u), dim3(64 * NW), 0, s, a, w,
                                     y, N, K, ks);
        // More row groups than compute units, one chunk per wavefront (K/32 ==
        // 8 x 16): 256 workgroups walk the row groups (LN), each splitting its
        // activations once instead of once per 16 rows, with the next group's
        // weights in flight while a group finishes (8 x 14336 x 4096: 19.8 ->
        // 10.9 us, 4 x 14336 x 4096: 16.0 -> 10.0, 1 x 14336 x 4096: 9.5 ->
        // 9.0). Non-temporal loads from M = 2 (1-3% there, 1.5% slower at M = 1
        // with partial-line loads), and always with whole lines (LA).
        if (splits == 1 && ch == 16 && ks == NW * 16 && grid > 256)
            return launch_kernel(k_gemv_stream<F, M, NW, 16, BF, 0, 16, (LA || M > 1), true, LA>,
                                 dim3(256u), dim3(64 * NW), 0, s, a, w, y, N, K, ks);
        // K = 8 x 8 blocks (2048): one 8-block chunk per wavefront rather than
        // 16-block chunks on half of them, looping over row groups as above
        // where there are more than 256 (8 x 11008 x 2048: 12.3 -> 6.6 us;
        // 8 x 4096 x 2048: 5.2 -> 4.45, 1 x 4096 x 2048: 3.50 -> 3.44).
        if (splits == 1 && ks == NW * 8 && grid > 256)
            return launch_kernel(k_gemv_stream<F, M, NW, 8, BF, 0, 16, (LA || M > 1), true, LA>,
                                 dim3(256u), dim3(64 * NW), 0, s, a, w, y, N, K, ks);
        if (splits == 1 && ks == NW * 8)
            return launch_kernel(k_gemv_stream<F, M, NW, 8, BF, 0, 16, true, false, LA>, g2,
                                 dim3(64 * NW), 0, s, a, w, y, N, K, ks);
        if (ch == 16) {
            if constexpr (GemvStreamCfg<F, M, NW, 16, BF>::AH == 1)
                if (al)
                    return launch_kernel(k_gemv_stream<F, M, NW, 16, BF, 1, 16, LA, false, LA>, g2, dim3(64 * NW),
                                         0, s, a, w, y, N, K, ks);
            if (al)
                return launch_kernel(k_gemv_stream<F, M, NW, 16, BF, 0, 16, LA, false, LA>, g2, dim3(64 * NW), 0, s,
                                     a, w, y, N, K, ks);
            return launch_kernel(k_gemv_stream<F, M, NW, 16, BF, 0, 16, true, false, LA>, g2, dim3(64 * NW),
                                 0, s, a, w, y, N, K, ks);
        }
        if (al)
            return launch_kernel(k_gemv_stream<F, M, NW, 8, BF, 1, 16, LA, false, LA>, g2, dim3(64 * NW), 0, s, a,
                                 w, y, N, K, ks);
        return launch_kernel(k_gemv_stream<F, M, NW, 8, BF, 0, 16, true, false, LA>, g2, dim3(64 * NW), 0, s, a, w,
                             y, N, K, ks);
    }
    return launch_kernel(k_gemv<F, M, BF>, dim3(grid), dim3(kGemvThreads), 0, s, a, w, y, N, K);
}

template <class F, int M, bool BF>
static hipError_t launch_gemv_m(const void *a, const uint8_t *w, float *y, int N, int K,
                                hipStream_t s, const q4v::GemvSplit &sp = {1, 0})
{
    if (gemv_rows_line_aligned<F>(w, K))
        return launch_gemv_m_la<F, M, BF, true>(a, w, y, N, K, s, sp);
    return launch_gemv_m_la<F, M, BF, false>(a, w, y, N, K, s, sp);
}

template <class F, bool BF>
static hipError_t launch_gemv_f(const void *a, const uint8_t *w, float *y, int M, int N, int K,
                                hipStream_t s)
{
    switch (M) {
    case 1: return launch_gemv_m<F, 1, BF>(a, w, y, N, K, s);
    case 2: return launch_gemv_m<F, 2, BF>(a, w, y, N, K, s);
    case 3: return launch_gemv_m<F, 3, BF>(a, w, y, N, K, s);
    case 4: return launch_gemv_m<F, 4, BF>(a, w, y, N, K, s);
    case 5: return launch_gemv_m<F, 5, BF>(a, w, y, N, K, s);
    case 6: return launch_gemv_m<F, 6, BF>(a, w, y, N, K, s);
    case 7: return launch_gemv_m<F, 7, BF>(a, w, y, N, K, s);
    case 8: return launch_gemv_m<F, 8, BF>(a, w, y, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M, int N,
                       int K, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemv_f<FmtQ8_0, false>(a, w, y, M, N, K, s);
    return launch_gemv_f<FmtQ4_0, false>(a, w, y, M, N, K, s);
}

hipError_t launch_gemv_bf16(WeightFormat fmt, const uint16_t *a, const uint8_t *w, float *y, int M,
                            int N, int K, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemv_f<FmtQ8_0, true>(a, w, y, M, N, K, s);
    return launch_gemv_f<FmtQ4_0, true>(a, w, y, M, N, K, s);
}

// ---------------------------------------------------------------------------
// Prepared activations. k_gemv_prep_ops makes, once, the A operands the
// streaming kernel would otherwise split in every workgroup: one workgroup per
// activation row finds the row's largest magnitude, takes the power of two p
// that puts the row's largest A value (2^kHiLog2 max |a| 2^p) in [2^14, 2^15)
// (row_scale_exp, as for a chunk), and writes for every block and lane group
// the hi and lo binary16 operands of A rows 2m and 2m + 1 in the kernel's slot
// order, then p. Operand (kb, g, i) sits at (kb * 4 + g) * 2M + i; the M
// exponents follow the nblk * 4 * 2M operands. A whole row shares one scale
// (the in-kernel split scales per chunk); elements far below the row maximum
// keep 2^-25 2^-p absolutely, as in the GEMM.
template <class F>
__global__ __launch_bounds__(256) void k_gemv_prep_ops(const float *__restrict__ a,
                                                      u32x4 *__restrict__ ops, int M, int K)
{
    __shared__ float s_mx[4];
    const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const float *row = a + (size_t)m * K;
    const float4 *row4 = reinterpret_cast<const float4 *>(row);
    float mx = 0.0f;
    for (int f = tid; f < K / 4; f += 256) {
        const float4 v = row4[f];
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    mx = wave_max_nonneg(mx);
    if (lane == 0)
        s_mx[tid >> 6] = mx;
    __syncthreads();
    const float am = fmaxf(fmaxf(s_mx[0], s_mx[1]), fmaxf(s_mx[2], s_mx[3]));
    const int p = row_scale_exp<F>(am);
    const float sh = ldexpf(1.0f, p), sl = (float)(1 << F::kHiLog2) * sh;
    const int nblk = K >> 5, NI = 2 * M;
    for (int t = tid; t < nblk * 4; t += 256) {
        const int kb = t >> 2, gg = t & 3;
        const float *blk = row + (size_t)kb * 32;
        const float4 L = *reinterpret_cast<const float4 *>(blk + F::a_lo(gg));
        const float4 H = *reinterpret_cast<const float4 *>(blk + F::a_hi(gg));
        const float v[8] = {L.x * sl, L.z * sl, L.y * sl, L.w * sl,
                            H.x * sh, H.z * sh, H.y * sh, H.w * sh};
        f16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            f16 hh, ll;
            split2(v[e], hh, ll);
            hi[e] = hh;
            lo[e] = ll;
        }
        u32x4 *dst = ops + ((size_t)kb * 4 + gg) * NI + 2 * m;
        dst[0] = bitcast<u32x4>(hi);
        dst[1] = bitcast<u32x4>(lo);
    }
    if (tid == 0)
        reinterpret_cast<int *>(ops + (size_t)nblk * 4 * NI)[m] = p;
}

template <class F, int M, bool LA>
static hipError_t launch_gemv_prepared_la(const void *prep, const uint8_t *w, float *y, int N,
                                          int K, hipStream_t s)
{
    constexpr int NW = kGemvStreamWaves;
    const int nblk = K / 32;
    const unsigned grid = (unsigned)((N + 15) / 16);
    // Non-temporal weight loads with whole-line loads (LA), or with one chunk
    // per wavefront and one workgroup per compute unit, as in launch_gemv_m;
    // row-group loops where there are more row groups than compute units, so each
    // workgroup loads the prepared operands once (8 x 14336 x 4096: 15.5 ->
    // 10.9 us, 1 x 14336 x 4096: 14.1 -> 9.9).
    // K = 2048: one 8-block chunk per wavefront (8 x 4096 x 2048: 4.15 ->
    // 3.8 us; with the row-group loops, 8 x 11008 x 2048: 8.3 -> 6.0).
    if (grid > 256 && nblk == NW * 8)
        return launch_kernel(k_gemv_stream<F, M, NW, 8, false, 2, 16, LA, true, LA>, dim3(256u),
                             dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
    if (nblk == NW * 8)
        return launch_kernel(k_gemv_stream<F, M, NW, 8, false, 2, 16, true, false, LA>, dim3(grid),
                             dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
    if (q4v::gemv_chunk_blocks(nblk, nblk) == 16) {
        if (grid > 256 && nblk == NW * 16)
            return launch_kernel(k_gemv_stream<F, M, NW, 16, false, 2, 16, LA, true, LA>, dim3(256u),
                                 dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
        if (grid <= 256 && nblk <= NW * 16)
            return launch_kernel(k_gemv_stream<F, M, NW, 16, false, 2, 16, true, false, LA>, dim3(grid),
                                 dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
        return launch_kernel(k_gemv_stream<F, M, NW, 16, false, 2, 16, LA, false, LA>, dim3(grid), dim3(64 * NW), 0,
                             s, prep, w, y, N, K, nblk);
    }
    if (grid <= 256 && nblk <= NW * 8)
        return launch_kernel(k_gemv_stream<F, M, NW, 8, false, 2, 16, true, false, LA>, dim3(grid),
                             dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
    return launch_kernel(k_gemv_stream<F, M, NW, 8, false, 2, 16, LA, false, LA>, dim3(grid),
                         dim3(64 * NW), 0, s, prep, w, y, N, K, nblk);
}

template <class F, int M>
static hipError_t launch_gemv_prepared_m(const void *prep, const uint8_t *w, float *y, int N, int K,
                                         hipStream_t s)
{
    if (gemv_rows_line_aligned<F>(w, K))
        return launch_gemv_prepared_la<F, M, true>(prep, w, y, N, K, s);
    return launch_gemv_prepared_la<F, M, false>(prep, w, y, N, K, s);
}

template <class F>
static hipError_t launch_gemv_prepared_f(const void *prep, const uint8_t *w, float *y, int M,
                                         int N, int K, hipStream_t s)
{
    switch (M) {
    case 1: return launch_gemv_prepared_m<F, 1>(prep, w, y, N, K, s);
    case 2: return launch_gemv_prepared_m<F, 2>(prep, w, y, N, K, s);
    case 3: return launch_gemv_prepared_m<F, 3>(prep, w, y, N, K, s);
    case 4: return launch_gemv_prepared_m<F, 4>(prep, w, y, N, K, s);
    case 5: return launch_gemv_prepared_m<F, 5>(prep, w, y, N, K, s);
    case 6: return launch_gemv_prepared_m<F, 6>(prep, w, y, N, K, s);
    case 7: return launch_gemv_prepared_m<F, 7>(prep, w, y, N, K, s);
    case 8: return launch_gemv_prepared_m<F, 8>(prep, w, y, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_prepare(WeightFormat fmt, const float *a, void *prep, int M, int K,
                               hipStream_t s)
{
    u32x4 *ops = static_cast<u32x4 *>(prep);
    if (fmt == WeightFormat::kQ8_0)
        return launch_kernel(k_gemv_prep_ops<FmtQ8_0>, dim3((unsigned)M), dim3(256), 0, s, a, ops,
                             M, K);
    return launch_kernel(k_gemv_prep_ops<FmtQ4_0>, dim3((unsigned)M), dim3(256), 0, s, a, ops, M,
                         K);
}

hipError_t launch_gemv_prepared(WeightFormat fmt, const void *prep, const uint8_t *w, float *y,
                                int M, int N, int K, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemv_prepared_f<FmtQ8_0>(prep, w, y, M, N, K, s);
    return launch_gemv_prepared_f<FmtQ4_0>(prep, w, y, M, N, K, s);
}

template <class F>
static hipError_t launch_gemv_splitk_f(const float *a, const uint8_t *w, float *y, int M, int N,
                                       int K, const q4v::GemvSplit &sp, float *part, hipStream_t s)
{
    float *out = sp.splits > 1 ? part : y;
    hipError_t e;
    switch (M) {
    case 1: e = launch_gemv_m<F, 1, false>(a, w, out, N, K, s, sp); break;
    case 2: e = launch_gemv_m<F, 2, false>(a, w, out, N, K, s, sp); break;
    case 3: e = launch_gemv_m<F, 3, false>(a, w, out, N, K, s, sp); break;
    case 4: e = launch_gemv_m<F, 4, false>(a, w, out, N, K, s, sp); break;
    case 5: e = launch_gemv_m<F, 5, false>(a, w, out, N, K, s, sp); break;
    case 6: e = launch_gemv_m<F, 6, false>(a, w, out, N, K, s, sp); break;
    case 7: e = launch_gemv_m<F, 7, false>(a, w, out, N, K, s, sp); break;
    case 8: e = launch_gemv_m<F, 8, false>(a, w, out, N, K, s, sp); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || sp.splits <= 1)
        return e;
    const long long n = (long long)M * N;
    return launch_kernel(k_gemv_split_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                         (const float *)part, y, n, sp.splits);
}

hipError_t launch_gemv_splitk(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M,
                              int N, int K, const q4v::GemvSplit &sp, void *workspace,
                              hipStream_t s)
{
    float *part = static_cast<float *>(workspace);
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemv_splitk_f<FmtQ8_0>(a, w, y, M, N, K, sp, part, s);
    return launch_gemv_splitk_f<FmtQ4_0>(a, w, y, M, N, K, sp, part, s);
}

// ---------------------------------------------------------------------------
// Q8_0-quantized activations. a_q is the [M, K/32] Q8_0 block stream of the
// activations (row m's blocks contiguous, in K order), so each block's dot
// product is an integer one, sum_j w_j q_j over the weight codes (q - 8 for
// Q4_0, the signed byte for Q8_0) and the activation codes, scaled by d_w d_a.
// * The integer sums run exactly on v_mfma_i32_16x16x32_i8 (K = 32, one
//   block): A rows are activation rows, B columns weight rows, so lane (j, g)
//   holds C rows 4g..4g+3 of weight row j, as in the f16 kernels.
// * The scale is applied in f32. d_w d_a has at most 22 significant bits and
//   stays normal, so it is exact; |sum| <= 2^19 converts exactly; one fused
//   multiply-add per block and C row adds sum d_w d_a to the chunk's partial
//   with one rounding. Partials: block -> chunk -> wavefront -> workgroup,
//   each level summed in a fixed order.
// * Operands of lane group g, eight signed bytes in slot order. Q4_0: qs dword
//   g; flipping bits 3 and 7 of each byte and masking nibbles gives bytes
//   16 (q - 8), the low nibbles (elements 4g..4g+3) after a 4-bit shift in
//   slots 0..3 and the high nibbles (elements 16+4g..16+4g+3) in slots 4..7.
//   The factor 16 comes out of d_w (a power of two: exact). The activation
//   operand takes its qs bytes 4g..4g+3 and 16+4g..16+4g+3. Q8_0: qs bytes
//   8g..8g+7 of both, unchanged.
// * Streaming form (K % 256 == 0): chunks of CH blocks dealt to the
//   wavefronts in turn, weights staged through LDS as in k_gemv_stream; the
//   chunk's M activation rows (CH * 34 bytes each, 16-byte aligned) are staged
//   beside them with 16-byte loads, and their scales are widened once per
//   chunk into an f32 [block][row] table.
// * LN (one chunk per wavefront, more row groups than compute units): the
//   workgroup walks row groups blockIdx.x, + gridDim.x, ... as k_gemv_stream
//   does; the chunk's activation blocks and scale table are staged once and
//   stay in LDS, and each group ends with its own reduction and store.

// Low and high nibbles of a Q4_0 qs dword as signed bytes 16 (q - 8).
__device__ __forceinline__ long q4_codes_x16(uint32_t x)
{
    const uint32_t t = x ^ 0x88888888u;
    const uint32_t lo = (t << 4) & 0xF0F0F0F0u;
    const uint32_t hi = t & 0xF0F0F0F0u;
    return (long)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ long pack_operand(uint32_t lo, uint32_t hi)
{
    return (long)(((uint64_t)hi << 32) | lo);
}

// Quant dword i of Q8_0 block B of a run of blocks that starts on a 4-byte
// boundary (the block's bytes 2 + 4i .. 5 + 4i).
template <int B>
__device__ __forceinline__ uint32_t q8_qs_dword(const uint32_t *row, int i)
{
    constexpr int o = kQ8Bytes * B + 2, i0 = o / 4, sh = o % 4;
    const uint32_t *p = row + i0 + i;
    if constexpr (sh != 0)
        return __builtin_amdgcn_alignbyte(p[1], p[0], 2u);
    else
        return p[0];
}

// Lane group g's activation operand from Q8_0 block B of a staged row, in the
// slot order of format F's weight operand.
template <class F, int B>
__device__ __forceinline__ long q8a_act_operand(const uint32_t *arow, int g)
{
    if constexpr (F::kBytes == kQ4Bytes)
        return pack_operand(q8_qs_dword<B>(arow, g), q8_qs_dword<B>(arow, 4 + g));
    else
        return pack_operand(q8_qs_dword<B>(arow, 2 * g), q8_qs_dword<B>(arow, 2 * g + 1));
}

// Lane group g's weight operand from block B of a staged weight row.
template <class F, int B>
__device__ __forceinline__ long q8a_weight_operand(const uint32_t *wrow, int g)
{
    uint32_t x[F::kQsDwords];
    read_qs<F, B>(wrow, g, x);
    if constexpr (F::kBytes == kQ4Bytes)
        return q4_codes_x16(x[0]);
    else
        return pack_operand(x[0], x[1]);
}

// d_w factor that undoes the weight operand's scaling (16 for Q4_0).
template <class F>
constexpr float q8a_weight_scale() { return F::kBytes == kQ4Bytes ? 0.0625f : 1.0f; }

template <class F, int M, int NW, int CH, bool NT = false, bool LN = false, bool LA = false>
__global__ __launch_bounds__(64 * NW) void k_gemv_q8a(const uint8_t *__restrict__ aq,
                                                     const uint8_t *__restrict__ w,
                                                     float *__restrict__ y, int N, int K)
{
    using C = GemvStreamCfg<F, M, NW, CH, false, 16, LA>;
    constexpr int NACC = M < 4 ? M : 4;           // C rows a lane keeps (activation rows 4g + r)
    constexpr int CPRA = CH * kQ8Bytes / 16;      // 16-byte columns of a chunk's activation row
    constexpr int NAE = M * CPRA;                 // ... of its M rows
    constexpr int NAL = (NAE + 63) / 64;          // ... per lane
    constexpr int RSA = CH * kQ8Bytes + 16;       // LDS bytes per staged activation row
    constexpr int ABYTES = M * RSA;
    constexpr int NDA = CH * M;                   // activation scales per chunk
    // Per wavefront: [staged weights | staged activations | scale table [CH][8]].
    constexpr int kLdsPerWave = C::WBYTES + ABYTES + CH * 8 * 4;
    static_assert(kLdsPerWave % 16 == 0, "16-byte aligned areas");
    __shared__ __attribute__((aligned(16))) uint8_t s_mem[NW * kLdsPerWave];
    __shared__ float s_part[LN ? 2 : 1][NW][M][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    int n0 = blockIdx.x * 16;
    const int nblk = K >> 5;
    const uint32_t row_bytes = (uint32_t)nblk * F::kBytes;
    const uint32_t arow_bytes = (uint32_t)nblk * kQ8Bytes;
    uint8_t *s_w = s_mem + wave * kLdsPerWave;
    uint8_t *s_act = s_w + C::WBYTES;
    float *s_da = reinterpret_cast<float *>(s_act + ABYTES);
    const int wb0 = wave * CH;                    // this wavefront's first chunk
    constexpr int kStride = NW * CH;              // ... and the step to its next

    // Weight loader role as in k_gemv_stream: eight lanes per row, eight rows
    // per load, then the tail columns.
    const int lrow = lane >> 3, lcol = lane & 7, trow = lane >> 2, tcol = lane & 3;
    uint32_t row_off0, row_off1, tail_off;
    auto set_rows = [&](int r0) __attribute__((always_inline)) {
        row_off0 = (uint32_t)min(r0 + lrow, N - 1) * row_bytes;
        row_off1 = (uint32_t)min(r0 + lrow + 8, N - 1) * row_bytes;
        tail_off = (uint32_t)min(r0 + trow, N - 1) * row_bytes +
                   16u * (uint32_t)(8 * C::NG + min(tcol, C::TC > 0 ? C::TC - 1 : 0));
    };
    set_rows(n0);

    u32x4 wreg[C::NLOAD];
    u32x4 areg[NAL];
    // Activation columns first (they drain first), then the weight columns.
    // Every lane issues every load; surplus lanes re-read the last activation
    // column and never store it.
    auto fetch_impl = [&](int cb0, auto acts_c) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < (decltype(acts_c)::value ? NAL : 0); ++r) {
            const int e = min(lane + 64 * r, NAE - 1);
            const int m = e / CPRA, col = e - m * CPRA;
            areg[r] = *reinterpret_cast<const u32x4 *>(
                aq + ((uint32_t)m * arow_bytes + (uint32_t)cb0 * kQ8Bytes + 16u * (uint32_t)col));
        }
        const uint32_t cbo = ((uint32_t)cb0 * F::kBytes) & (LA ? ~127u : ~0u);   // LA: from the chunk's first line
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2 * C::NG; ++i) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                w + ((i & 1 ? row_off1 : row_off0) + cbo + 16u * (uint32_t)(lcol + 8 * (i >> 1))));
            wreg[i] = NT ? __builtin_nontemporal_load(src) : *src;
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (C::TC > 0)
        {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(w + (tail_off + cbo));
            wreg[2 * C::NG] = NT ? __builtin_nontemporal_load(src) : *src;
        }
        asm volatile("" ::"s"(w), "s"(aq) : "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto fetch = [&](int cb0) __attribute__((always_inline)) { fetch_impl(cb0, std::true_type{}); };
    auto fetch_w = [&](int cb0) __attribute__((always_inline)) { fetch_impl(cb0, std::false_type{}); };
    // A wavefront without blocks fetches the row's last chunk and never reads it.
    fetch(min(wb0, nblk - CH));

    const uint32_t *arow32 = reinterpret_cast<const uint32_t *>(s_act + min(j, M - 1) * RSA);
    const uint8_t *wrow = s_w + j * C::RS;
    const float *da_lane = s_da + 4 * min(g, 1);
    const i32x4 zero4 = {0, 0, 0, 0};
    float ysum[NACC];
#pragma unroll
    for (int r = 0; r < NACC; ++r)
        ysum[r] = 0.0f;

    // Epilogue of one row group: wavefront partials into LDS (buffer buf),
    // then summed in wavefront order and stored.
    auto write_out = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < NACC; ++r) {
            const int m = 4 * g + r;
            if (m < M)
                s_part[buf][wave][m][j] = ysum[r];
            ysum[r] = 0.0f;
        }
        __syncthreads();
        if (tid < M * 16) {
            const int m = tid >> 4, jj = tid & 15, n = n0 + jj;
            float sum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww)
                sum += s_part[buf][ww][m][jj];
            if (n < N)
                y[(size_t)m * N + n] = sum;
        }
    };
    // LN: this workgroup's row group (it walks groups blockIdx.x, + gridDim.x,
    // ...); the chunk's activation blocks and scale table stay in LDS.
    int rg = blockIdx.x, it = 0;
    for (int cb0 = wb0; cb0 < nblk; cb0 += LN ? 0 : kStride) {
        const bool more = LN ? (rg + (int)gridDim.x) * 16 < N : cb0 + kStride < nblk;
        if (!LN || it == 0) {
#pragma unroll
            for (int r = 0; r < NAL; ++r) {
                const int e = lane + 64 * r;
                if (e < NAE) {
                    const int m = e / CPRA, col = e - m * CPRA;
                    *reinterpret_cast<u32x4 *>(s_act + m * RSA + 16 * col) = areg[r];
                }
            }
            wave_lds_sync();
#pragma unroll
            for (int r = 0; r < (NDA + 63) / 64; ++r) {
                const int t = lane + 64 * r;
                if (t < NDA) {
                    const int b = t / M, m = t - b * M;
                    s_da[b * 8 + m] = f16_bits_to_f32(
                        *reinterpret_cast<const uint16_t *>(s_act + m * RSA + kQ8Bytes * b));
                }
            }
        }
        float acc[NACC];
#pragma unroll
        for (int r = 0; r < NACC; ++r)
            acc[r] = 0.0f;
        // LA: the chunk starts (cb0 kBytes) mod 128 bytes into the staged lines.
        const uint32_t *wrow32 = reinterpret_cast<const uint32_t *>(
            wrow + (LA ? (((uint32_t)cb0 * F::kBytes) & 127u) : 0u));
        auto stage = [&](auto i0_c, auto i1_c) __attribute__((always_inline)) {
            constexpr int I0 = decltype(i0_c)::value, I1 = decltype(i1_c)::value;
#pragma unroll
            for (int i = I0; i < I1; ++i) {
                if (i < C::RH * C::NG)
                    *reinterpret_cast<u32x4 *>(s_w + (lrow + 8 * (i % C::RH)) * C::RS +
                                               16 * (lcol + 8 * (i / C::RH))) = wreg[i];
                else if (tcol < C::TC)
                    *reinterpret_cast<u32x4 *>(s_w + trow * C::RS + 16 * (8 * C::NG + tcol)) = wreg[i];
            }
        };
        // All integer MFMAs of a part are issued before its scale FMAs.
        auto contract = [&](auto b0_c, auto b1_c) __attribute__((always_inline)) {
            constexpr int B0 = decltype(b0_c)::value, B1 = decltype(b1_c)::value;
            i32x4 Dv[B1 - B0];
            float dw[B1 - B0];
            static_for<B0, B1>([&](auto b_c) __attribute__((always_inline)) {
                constexpr int b = decltype(b_c)::value;
                const long bw = q8a_weight_operand<F, b>(wrow32, g);
                const long av = q8a_act_operand<F, b>(arow32, g);
                dw[b - B0] = f16_bits_to_f32(read_d_bits<F, b>(wrow32)) * q8a_weight_scale<F>();
                Dv[b - B0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bw, zero4, 0, 0, 0);
            });
#pragma unroll
            for (int u = 0; u < B1 - B0; ++u) {
                // Only the NACC scales this lane uses: whole 16-byte reads of the
                // table would be hoisted for every block of the chunk and hold
                // 64 VGPRs at M = 1.
                float da[NACC];
#pragma unroll
                for (int r = 0; r < NACC; ++r)
                    da[r] = da_lane[(B0 + u) * 8 + r];
#pragma unroll
                for (int r = 0; r < NACC; ++r)
                    acc[r] = fmaf(dw[u] * da[r], (float)Dv[u][r], acc[r]);
            }
#pragma unroll
            for (int u = 0; u < B1 - B0; ++u)
                asm volatile("" ::"v"(Dv[u]));
        };
        for_each_part<C::NPART>([&](auto p_c) __attribute__((always_inline)) {
            constexpr int P = decltype(p_c)::value;
            constexpr int B0 = P * CH / C::NPART, B1 = (P + 1) * CH / C::NPART;
            constexpr int L0 = C::loads_for(B0), L1 = C::loads_for(B1);
            stage(std::integral_constant<int, L0>{}, std::integral_constant<int, L1>{});
            auto run_part = [&]() __attribute__((always_inline)) {
                wave_lds_sync();
                contract(std::integral_constant<int, B0>{}, std::integral_constant<int, B1>{});
            };
            if constexpr (P < C::NPART - 1) {
                run_part();
            } else if (LN && more) {
                // Every weight register of this group is staged: the next
                // group's loads for the same chunk, then this group's last part.
                set_rows((rg + (int)gridDim.x) * 16);
                fetch_w(cb0);
                run_part();
            } else if (more) {
                fetch(cb0 + kStride);   // every register of this chunk is staged
                run_part();
            } else {
                run_part();
            }
        });
#pragma unroll
        for (int r = 0; r < NACC; ++r)
            ysum[r] += acc[r];
        wave_lds_sync();   // this chunk's LDS reads precede the next chunk's writes
        if constexpr (LN) {
            write_out(it & 1);
            if (!more)
                break;
            rg += (int)gridDim.x;
            ++it;
            n0 = rg * 16;
        }
    }
    if constexpr (!LN)
        write_out(0);
}


// General shapes (K % 256 != 0, or offsets beyond 31 bits): the same
// arithmetic with each lane loading its operands and scales from global memory
// (2-byte aligned dword loads); wavefront w takes blocks w, w + 8, ...
template <class F, int M>
__global__ __launch_bounds__(kGemvThreads) void k_gemv_q8a_any(const uint8_t *__restrict__ aq,
                                                              const uint8_t *__restrict__ w,
                                                              float *__restrict__ y, int N, int K)
{
    constexpr int NW = kGemvWaves;
    constexpr int NACC = M < 4 ? M : 4;
    __shared__ float s_part[NW][M][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int nblk = K >> 5;
    const uint8_t *wrow = w + (size_t)min(n0 + j, N - 1) * (size_t)nblk * F::kBytes;
    const uint8_t *arow = aq + (size_t)min(j, M - 1) * (size_t)nblk * kQ8Bytes;
    const uint8_t *drow[NACC];
#pragma unroll
    for (int r = 0; r < NACC; ++r)
        drow[r] = aq + (size_t)min(4 * g + r, M - 1) * (size_t)nblk * kQ8Bytes;
    const i32x4 zero4 = {0, 0, 0, 0};
    float acc[NACC];
#pragma unroll
    for (int r = 0; r < NACC; ++r)
        acc[r] = 0.0f;
    for (int b = wave; b < nblk; b += NW) {
        const uint8_t *wb = wrow + (size_t)b * F::kBytes;
        const uint8_t *ab = arow + (size_t)b * kQ8Bytes + 2;
        uint32_t x[F::kQsDwords];
        load_qs<F>(wb, g, x);
        long bw, av;
        if constexpr (F::kBytes == kQ4Bytes) {
            bw = q4_codes_x16(x[0]);
            av = pack_operand(load_u32_unaligned(ab + 4 * g), load_u32_unaligned(ab + 16 + 4 * g));
        } else {
            bw = pack_operand(x[0], x[1]);
            av = pack_operand(load_u32_unaligned(ab + 8 * g), load_u32_unaligned(ab + 8 * g + 4));
        }
        const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bw, zero4, 0, 0, 0);
        const float dw = f16_bits_to_f32(load_u16(wb)) * q8a_weight_scale<F>();
#pragma unroll
        for (int r = 0; r < NACC; ++r)
            acc[r] = fmaf(dw * f16_bits_to_f32(load_u16(drow[r] + (size_t)b * kQ8Bytes)),
                          (float)D[r], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < NACC; ++r) {
        const int m = 4 * g + r;
        if (m < M)
            s_part[wave][m][j] = acc[r];
    }
    __syncthreads();
    if (tid < M * 16) {
        const int m = tid >> 4, jj = tid & 15, n = n0 + jj;
        float sum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww)
            sum += s_part[ww][m][jj];
        if (n < N)
            y[(size_t)m * N + n] = sum;
    }
}

template <class F, int M, bool LA>
static hipError_t launch_gemv_q8a_la(const uint8_t *aq, const uint8_t *w, float *y, int N, int K,
                                     hipStream_t s)
{
    constexpr int NW = kGemvStreamWaves;
    const unsigned grid = (unsigned)((N + 15) / 16);
    if (q4v::gemv_q8a_streams(M, N, K, F::kBytes)) {
        const int nblk = K / 32;
        // 16-block chunks, except where there are more workgroups than compute
        // units and M > 1: those kernels need more than 128 VGPRs, so one
        // workgroup holds a compute unit, while the 8-block ones (under 100)
        // let two or more share it and overlap one's loads with another's work.
        // Non-temporal weight loads as in launch_gemv_m: with whole-line
        // loads (LA) everywhere (1 x 14336 x 4096 9.08 -> 8.59 us, Q8_0
        // weights 1 x 4096 x 4096 5.55 -> 5.12, 8 x 11008 x 2048 6.69 ->
        // 6.15), otherwise one chunk per wavefront and one workgroup per
        // compute unit.
        // More row groups than compute units and one 16-block chunk per
        // wavefront, from two activation rows: 256 workgroups walk the row
        // groups, staging each chunk's activation blocks and scales once (as
        // launch_gemv_m; 8 x 14336 x 4096: 13.6 -> 11.4 us, 8 x 8192 x 4096:
        // 8.2 -> 7.2; one row: 9.1 -> 9.5, so not there). Non-temporal loads
        // with whole lines, else for Q4_0 weights only (Q8_0 8 x 14336 x 4096
        // with partial lines: 15.4 us plain, 16.3; whole lines and
        // non-temporal: 14.4).
        if constexpr (M > 1)
            if (q4v::gemv_chunk_blocks(nblk, nblk) == 16 && grid > 256 && nblk == NW * 16)
                return launch_kernel(k_gemv_q8a<F, M, NW, 16, LA || F::kBytes == kQ4Bytes, true, LA>,
                                     dim3(256u), dim3(64 * NW), 0, s, aq, w, y, N, K);
        // K = 2048: one 8-block chunk per wavefront, with the row-group loops
        // from two rows on wide grids (8 x 11008 x 2048: 7.25 -> 6.7 us).
        if constexpr (M > 1)
            if (grid > 256 && nblk == NW * 8)
                return launch_kernel(k_gemv_q8a<F, M, NW, 8, LA || F::kBytes == kQ4Bytes, true, LA>,
                                     dim3(256u), dim3(64 * NW), 0, s, aq, w, y, N, K);
        if (grid <= 256 && nblk == NW * 8)
            return launch_kernel(k_gemv_q8a<F, M, NW, 8, true, false, LA>, dim3(grid), dim3(64 * NW), 0, s,
                                 aq, w, y, N, K);
        if (q4v::gemv_chunk_blocks(nblk, nblk) == 16 && grid <= 256 && nblk <= NW * 16)
            return launch_kernel(k_gemv_q8a<F, M, NW, 16, true, false, LA>, dim3(grid), dim3(64 * NW), 0, s,
                                 aq, w, y, N, K);
        if (q4v::gemv_chunk_blocks(nblk, nblk) == 16 && (grid <= 256 || M == 1))
            return launch_kernel(k_gemv_q8a<F, M, NW, 16, LA, false, LA>, dim3(grid), dim3(64 * NW), 0, s, aq, w,
                                 y, N, K);
        return launch_kernel(k_gemv_q8a<F, M, NW, 8, LA, false, LA>, dim3(grid), dim3(64 * NW), 0, s, aq, w, y,
                             N, K);
    }
    return launch_kernel(k_gemv_q8a_any<F, M>, dim3(grid), dim3(kGemvThreads), 0, s, aq, w, y, N,
                         K);
}

template <class F, int M>
static hipError_t launch_gemv_q8a_m(const uint8_t *aq, const uint8_t *w, float *y, int N, int K,
                                    hipStream_t s)
{
    if (gemv_rows_line_aligned<F>(w, K))
        return launch_gemv_q8a_la<F, M, true>(aq, w, y, N, K, s);
    return launch_gemv_q8a_la<F, M, false>(aq, w, y, N, K, s);
}

template <class F>
static hipError_t launch_gemv_q8a_f(const uint8_t *aq, const uint8_t *w, float *y, int M, int N,
                                    int K, hipStream_t s)
{
    switch (M) {
    case 1: return launch_gemv_q8a_m<F, 1>(aq, w, y, N, K, s);
    case 2: return launch_gemv_q8a_m<F, 2>(aq, w, y, N, K, s);
    case 3: return launch_gemv_q8a_m<F, 3>(aq, w, y, N, K, s);
    case 4: return launch_gemv_q8a_m<F, 4>(aq, w, y, N, K, s);
    case 5: return launch_gemv_q8a_m<F, 5>(aq, w, y, N, K, s);
    case 6: return launch_gemv_q8a_m<F, 6>(aq, w, y, N, K, s);
    case 7: return launch_gemv_q8a_m<F, 7>(aq, w, y, N, K, s);
    case 8: return launch_gemv_q8a_m<F, 8>(aq, w, y, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_q8a(WeightFormat fmt, const uint8_t *a_q, const uint8_t *w, float *y, int M,
                           int N, int K, hipStream_t s)
{
    if (fmt == WeightFormat::kQ8_0)
        return launch_gemv_q8a_f<FmtQ8_0>(a_q, w, y, M, N, K, s);
    return launch_gemv_q8a_f<FmtQ4_0>(a_q, w, y, M, N, K, s);
}

}  // namespace q4k
