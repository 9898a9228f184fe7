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
int check_product(const float *a, const void *w, size_t w_bytes, const float *y,
                  int M, int N, int K, int max_rows, size_t block_bytes, bool *empty);
int check_quantize(const float *x, size_t n_elems, const void *out, size_t out_bytes,
                   size_t block_bytes, bool *empty);

// True when q4_gemm / q8_gemm take the split-activation path for this K (the
// path that needs a workspace). The GEMM launcher branches on the same
// predicate.
inline bool gemm_splits_activations(int K) { return K > 0 && K % 64 == 0; }

// Workspace bytes q4_gemm and q8_gemm need: 0 when none (no split path, or an empty or
// invalid shape), SIZE_MAX when the size does not fit in size_t.
size_t gemm_workspace_bytes(int M, int N, int K);

// Checks of a GEMM workspace, after check_product has passed for a
// non-empty problem: size, then NULL, alignment and overlap with a, w and y.
int check_workspace(const float *a, const void *w, size_t w_bytes, const float *y, int M, int N,
                    int K, const void *ws, size_t ws_bytes);

bool aligned16(const void *p);
bool overlaps(Span a, Span b);

}  // namespace q4v
