// Argument validation for the C ABI in include/q4.h. Pure host C++ with no HIP
// dependency: every check here runs before anything is launched.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace q4v {

// Byte extent [p, p + n) of one argument.
struct Span {
    const void *p;
    size_t n;
};

// Each returns Q4_OK or a Q4_ERR_* code; *empty is set when the problem has no
// work (then nothing is to be launched and the pointers were not inspected).
// block_bytes: 18 for Q4_0 streams, 34 for Q8_0 streams.
int check_dequant(const void *w, size_t w_bytes, const float *out, size_t out_elems,
                  size_t block_bytes, bool *empty);
// a_elem: bytes of one activation (4 for f32, 2 for bfloat16).
int check_product(const void *a, size_t a_elem, const void *w, size_t w_bytes, const float *y,
                  int M, int N, int K, int max_rows, size_t block_bytes, bool *empty);
int check_quantize(const float *x, size_t n_elems, const void *out, size_t out_bytes,
                   size_t block_bytes, bool *empty);

// True when the GEMMs take the split-activation path for this K (with
// M N < 2^31, the split kernel's 32-bit output offsets). The GEMM launchers
// branch on the same predicate.
// K <= 2^22 keeps every byte offset of the split kernel's buffer loads within
// 32 bits.
inline bool gemm_splits_activations(int K) { return K > 0 && K % 64 == 0 && K <= (1 << 22); }

// Workspace bytes the f32 GEMM (q4_gemm_ws, q8_gemm_ws) needs: the row
// exponents, then on the split path ceil(M / 128) * 128 * K * 4 bytes of
// two-term operands. 0 for an empty or invalid shape, SIZE_MAX when the size
// does not fit in size_t.
size_t gemm_workspace_bytes(int M, int N, int K);

// The bfloat16 GEMM's split path: K % 64 == 0 and M N < 2^31 (the split
// kernel's 32-bit output offsets). Otherwise it takes the general kernel.
inline bool gemm_bf16_splits(int M, int N, int K)
{
    return gemm_splits_activations(K) && (long long)M * N < (1LL << 31);
}

// The streaming GEMV kernel's shapes: 16-byte aligned weight rows (K % 256 ==
// 0) and 32-bit byte offsets into W and a. Other shapes take the general GEMV
// kernel.
inline bool gemv_streams(int M, int N, int K, size_t block_bytes, size_t a_elem)
{
    return K > 0 && K % 256 == 0 && (size_t)N * (size_t)(K / 32) * block_bytes < ((size_t)1 << 31) &&
           (size_t)M * (size_t)K * a_elem < ((size_t)1 << 31);
}

// A K split of the decode GEMV: `splits` workgroups per 16 output columns, each
// over ks consecutive blocks (a multiple of 8; the last split takes the rest).
struct GemvSplit {
    int splits;
    int ks;
};

// Blocks per chunk of the streaming GEMV for splits of ks blocks (the last one
// kl): 16 when both divide by 16, else 8 (K % 256 == 0 makes every split a
// multiple of 8).
inline int gemv_chunk_blocks(int ks, int kl) { return (ks % 16 == 0 && kl % 16 == 0) ? 16 : 8; }

// Chunks the busiest wavefront of the streaming GEMV walks in turn when K is
// not split (the chunks of a row are dealt to its 8 wavefronts in turn).
inline int gemv_chunks_per_wave(int nblk)
{
    const int chunks = nblk / gemv_chunk_blocks(nblk, nblk);
    return (chunks + 7) / 8;
}

// The split a q4_gemv_splitk / q8_gemv_splitk call uses: `requested` splits,
// at most one per 8 blocks, and 1 (no split) for shapes off the streaming
// kernel or invalid ones. 0 asks for the library's choice: no split unless
// each wavefront would walk at least 3 chunks in turn (below that, the extra
// kernel that adds the partials costs more than the split saves), else
// ceil(256 / ceil(N / 16)) splits (enough workgroups for 256 compute units),
// at most one per 64 blocks.
inline GemvSplit gemv_split_plan(int M, int N, int K, int requested, size_t block_bytes)
{
    if (M <= 0 || N <= 0 || requested < 0 || !gemv_streams(M, N, K, block_bytes, 4))
        return {1, 0};
    const int nblk = K / 32, groups = (N + 15) / 16;
    int want = requested;
    if (want == 0) {
        want = (256 + groups - 1) / groups;
        want = want < nblk / 64 ? want : nblk / 64;
        if (gemv_chunks_per_wave(nblk) < 3)
            want = 1;
    }
    want = want < nblk / 8 ? want : nblk / 8;
    if (want <= 1)
        return {1, nblk};
    const int ks = ((nblk + want - 1) / want + 7) & ~7;
    return {(nblk + ks - 1) / ks, ks};
}

// Bytes of a GEMV's prepared activations (q4_gemv_prepare): the two-term A
// operands of every block, K/32 * 4 * 2M * 16 bytes, then M int32 exponents
// padded to 16 bytes. 0 for M outside [1, 8] or K not a positive multiple of
// 256 (the prepared GEMV runs the streaming kernel only).
inline size_t gemv_prepare_bytes(int M, int K)
{
    if (M < 1 || M > 8 || K <= 0 || K % 256 != 0)
        return 0;
    return (size_t)(K / 32) * 4 * 2 * (size_t)M * 16 + ((size_t)M * 4 + 15) / 16 * 16;
}

// Checks of q4_gemv_prepare (a [M, K] f32 -> prep) and of the prepared GEMV
// (prep, W -> y): shape (1 <= M <= 8, K % 256 == 0, the streaming kernel's
// offset limits), sizes (prep_bytes >= gemv_prepare_bytes), then NULL,
// alignment and overlap, as check_product. M == 0 (or N == 0) is empty.
int check_gemv_prepare(const float *a, int M, int K, const void *prep, size_t prep_bytes,
                       bool *empty);
int check_gemv_prepared(const void *prep, size_t prep_bytes, const void *w, size_t w_bytes,
                        const float *y, int M, int N, int K, size_t block_bytes, bool *empty);

// Workspace bytes of a K-split GEMV: splits * M * N f32 partials, or 0 when the
// call does not split (then the workspace is not used).
size_t gemv_splitk_workspace_bytes(int M, int N, int K, int requested, size_t block_bytes);

// Bytes at the start of every GEMM workspace that hold the per-row exponents
// (M int32, padded to 256 bytes); the activation operands follow.
inline size_t gemm_row_exp_bytes(int M) { return ((size_t)M * 4 + 255) / 256 * 256; }

// Workspace bytes q4_gemm_bf16 and q8_gemm_bf16 need: the row exponents, then
// ceil(M / 128) * 128 * K binary16 operands on the split path or M * K f32
// otherwise. 0 for an empty or invalid shape, SIZE_MAX when it does not fit.
size_t gemm_bf16_workspace_bytes(int M, int N, int K);

// Checks of a GEMM workspace of `need` bytes (the shape's workspace_bytes
// function), after check_product has passed for a non-empty problem: size,
// then NULL, alignment and overlap with a (a_elem bytes per element), w and y.
int check_workspace(size_t need, const void *a, size_t a_elem, const void *w, size_t w_bytes,
                    const float *y, int M, int N, int K, const void *ws, size_t ws_bytes);
// The same with the activations' byte count given directly.
int check_workspace_span(size_t need, const void *a, size_t a_bytes, const void *w, size_t w_bytes,
                         const float *y, int M, int N, const void *ws, size_t ws_bytes);

// The products over Q8_0-quantized activations (q4_gemv_q8a, q4_gemm_q8a and
// the Q8_0-weight forms): a_q is the [M, K/32] Q8_0 block stream of the
// activations, a_bytes == M (K/32) 34, then as check_product (at most
// max_rows rows when max_rows > 0; M == 0 or N == 0 is empty).
int check_product_q8a(const void *a_q, size_t a_bytes, const void *w, size_t w_bytes,
                      const float *y, int M, int N, int K, int max_rows, size_t block_bytes,
                      bool *empty);

// Workspace bytes q4_gemm_q8a and q8_gemm_q8a need: the row exponents (as the
// bfloat16 GEMM's), then the activations as the f32 GEMM's split operands on
// its split path (ceil(M / 128) * 128 * K * 4 bytes) or as scaled f32 values
// otherwise (M * K * 4). 0 for an empty or invalid shape, SIZE_MAX when it
// does not fit.
size_t gemm_q8a_workspace_bytes(int M, int N, int K);

// Its streaming kernel's shapes: 16-byte aligned weight and activation rows
// (K % 256 == 0) and byte offsets into W and a_q below 2^31. Other shapes take
// its general kernel.
inline bool gemv_q8a_streams(int M, int N, int K, size_t block_bytes)
{
    return K > 0 && K % 256 == 0 && (size_t)N * (size_t)(K / 32) * block_bytes < ((size_t)1 << 31) &&
           (size_t)M * (size_t)(K / 32) * 34 < ((size_t)1 << 31);
}

bool aligned16(const void *p);
bool overlaps(Span a, Span b);

}  // namespace q4v
