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

// True when q4_gemm / q8_gemm take the split-activation path for this K (the
// path that needs a workspace). The GEMM launcher branches on the same
// predicate.
// K <= 2^22 keeps every byte offset of the split kernel's buffer loads within
// 32 bits.
inline bool gemm_splits_activations(int K) { return K > 0 && K % 64 == 0 && K <= (1 << 22); }

// Workspace bytes q4_gemm and q8_gemm need: 0 when none (no split path, or an empty or
// invalid shape), SIZE_MAX when the size does not fit in size_t.
size_t gemm_workspace_bytes(int M, int N, int K);

// The bfloat16 GEMM's split path: K % 64 == 0 and M N < 2^31 (the split
// kernel's 32-bit output offsets). Otherwise it takes the general kernel.
inline bool gemm_bf16_splits(int M, int N, int K)
{
    return gemm_splits_activations(K) && (long long)M * N < (1LL << 31);
}

// Bytes at the start of a bfloat16 GEMM workspace that hold the per-row
// exponents (M int32, padded to 256 bytes); the activation operands follow.
inline size_t gemm_bf16_row_exp_bytes(int M) { return ((size_t)M * 4 + 255) / 256 * 256; }

// Workspace bytes q4_gemm_bf16 and q8_gemm_bf16 need: the row exponents, then
// ceil(M / 128) * 128 * K binary16 operands on the split path or M * K f32
// otherwise. 0 for an empty or invalid shape, SIZE_MAX when it does not fit.
size_t gemm_bf16_workspace_bytes(int M, int N, int K);

// Checks of a GEMM workspace of `need` bytes (the shape's workspace_bytes
// function), after check_product has passed for a non-empty problem: size,
// then NULL, alignment and overlap with a (a_elem bytes per element), w and y.
int check_workspace(size_t need, const void *a, size_t a_elem, const void *w, size_t w_bytes,
                    const float *y, int M, int N, int K, const void *ws, size_t ws_bytes);

bool aligned16(const void *p);
bool overlaps(Span a, Span b);

}  // namespace q4v
