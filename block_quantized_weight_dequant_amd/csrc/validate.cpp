// Argument validation for the C ABI (include/q4.h). The order of the checks is
// fixed: shape, then sizes, then the empty case, then pointers (NULL, 16-byte
// alignment, output/input overlap). Nothing here touches device memory.
#include "validate.h"

#include "q4.h"

namespace q4v {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(Span a, Span b)
{
    if (a.n == 0 || b.n == 0)
        return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    // a0 + a.n cannot wrap for a real allocation; the compare stays in unsigned.
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

static bool mul_ok(size_t x, size_t y, size_t *r) { return !__builtin_mul_overflow(x, y, r); }

int check_dequant(const void *w, size_t w_bytes, const float *out, size_t out_elems,
                  size_t block_bytes, bool *empty)
{
    *empty = false;
    if (w_bytes % block_bytes != 0)
        return Q4_ERR_SIZE;
    size_t nb = w_bytes / block_bytes, want = 0, out_bytes = 0;
    if (!mul_ok(nb, 32, &want) || out_elems != want)
        return Q4_ERR_SIZE;
    if (!mul_ok(out_elems, sizeof(float), &out_bytes))
        return Q4_ERR_SIZE;
    if (nb == 0) {
        *empty = true;
        return Q4_OK;
    }
    if (!w || !out)
        return Q4_ERR_NULL;
    if (!aligned16(w) || !aligned16(out))
        return Q4_ERR_ALIGN;
    if (overlaps({w, w_bytes}, {out, out_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

int check_product(const void *a, size_t a_elem, const void *w, size_t w_bytes, const float *y,
                  int M, int N, int K, int max_rows, size_t block_bytes, bool *empty)
{
    *empty = false;
    if (M < 0 || N < 0 || K < 32 || K % 32 != 0)
        return Q4_ERR_SHAPE;
    if (max_rows > 0 && M > max_rows)
        return Q4_ERR_SHAPE;
    size_t row_bytes = (size_t)(K / 32) * block_bytes, w_want = 0, a_bytes = 0, y_bytes = 0;
    if (!mul_ok((size_t)N, row_bytes, &w_want) || w_bytes != w_want)
        return Q4_ERR_SIZE;
    if (!mul_ok((size_t)M, (size_t)K, &a_bytes) || !mul_ok(a_bytes, a_elem, &a_bytes))
        return Q4_ERR_SIZE;
    if (!mul_ok((size_t)M, (size_t)N, &y_bytes) || !mul_ok(y_bytes, sizeof(float), &y_bytes))
        return Q4_ERR_SIZE;
    if (M == 0 || N == 0) {
        *empty = true;
        return Q4_OK;
    }
    if (!a || !w || !y)
        return Q4_ERR_NULL;
    if (!aligned16(a) || !aligned16(w) || !aligned16(y))
        return Q4_ERR_ALIGN;
    if (overlaps({y, y_bytes}, {a, a_bytes}) || overlaps({y, y_bytes}, {w, w_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

int check_product_q8a(const void *a_q, size_t a_bytes, const void *w, size_t w_bytes,
                      const float *y, int M, int N, int K, int max_rows, size_t block_bytes,
                      bool *empty)
{
    *empty = false;
    if (M < 0 || N < 0 || K < 32 || K % 32 != 0 || (max_rows > 0 && M > max_rows))
        return Q4_ERR_SHAPE;
    size_t w_want = 0, a_want = 0, y_bytes = 0;
    if (!mul_ok((size_t)N, (size_t)(K / 32) * block_bytes, &w_want) || w_bytes != w_want)
        return Q4_ERR_SIZE;
    if (!mul_ok((size_t)M, (size_t)(K / 32) * 34, &a_want) || a_bytes != a_want)
        return Q4_ERR_SIZE;
    if (!mul_ok((size_t)M, (size_t)N, &y_bytes) || !mul_ok(y_bytes, sizeof(float), &y_bytes))
        return Q4_ERR_SIZE;
    if (M == 0 || N == 0) {
        *empty = true;
        return Q4_OK;
    }
    if (!a_q || !w || !y)
        return Q4_ERR_NULL;
    if (!aligned16(a_q) || !aligned16(w) || !aligned16(y))
        return Q4_ERR_ALIGN;
    if (overlaps({y, y_bytes}, {a_q, a_bytes}) || overlaps({y, y_bytes}, {w, w_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

int check_quantize(const float *x, size_t n_elems, const void *out, size_t out_bytes,
                   size_t block_bytes, bool *empty)
{
    *empty = false;
    if (n_elems % 32 != 0)
        return Q4_ERR_SHAPE;
    size_t want = 0, x_bytes = 0;
    if (!mul_ok(n_elems / 32, block_bytes, &want) || out_bytes != want)
        return Q4_ERR_SIZE;
    if (!mul_ok(n_elems, sizeof(float), &x_bytes))
        return Q4_ERR_SIZE;
    if (n_elems == 0) {
        *empty = true;
        return Q4_OK;
    }
    if (!x || !out)
        return Q4_ERR_NULL;
    if (!aligned16(x) || !aligned16(out))
        return Q4_ERR_ALIGN;
    if (overlaps({x, x_bytes}, {out, out_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

size_t gemm_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K < 32 || K % 32 != 0)
        return 0;
    const size_t r = gemm_row_exp_bytes(M);
    // The split path also needs M N < 2^31 (its 32-bit output offsets); larger
    // outputs take the general kernel, which needs the row exponents only.
    if (!gemm_splits_activations(K) || (long long)M * N >= (1LL << 31))
        return r;
    // Rows are padded to whole 128-row tiles; hi and lo binary16 per element.
    size_t mp = ((size_t)M + 127) / 128 * 128, n = 0;
    if (!mul_ok(mp, (size_t)K, &n) || !mul_ok(n, 4, &n))
        return SIZE_MAX;
    return n > SIZE_MAX - r ? SIZE_MAX : n + r;
}

int check_gemv_prepare(const float *a, int M, int K, const void *prep, size_t prep_bytes,
                       bool *empty)
{
    *empty = false;
    if (M < 0 || M > Q4_GEMV_MAX_ROWS || K < 256 || K % 256 != 0)
        return Q4_ERR_SHAPE;
    if (M == 0) {
        *empty = true;
        return Q4_OK;
    }
    const size_t need = gemv_prepare_bytes(M, K);
    if (prep_bytes < need)
        return Q4_ERR_SIZE;
    if (!a || !prep)
        return Q4_ERR_NULL;
    if (!aligned16(a) || !aligned16(prep))
        return Q4_ERR_ALIGN;
    if (overlaps({prep, need}, {a, (size_t)M * (size_t)K * sizeof(float)}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

int check_gemv_prepared(const void *prep, size_t prep_bytes, const void *w, size_t w_bytes,
                        const float *y, int M, int N, int K, size_t block_bytes, bool *empty)
{
    *empty = false;
    if (M < 0 || M > Q4_GEMV_MAX_ROWS || N < 0 || K < 256 || K % 256 != 0)
        return Q4_ERR_SHAPE;
    size_t w_want = 0, y_bytes = 0;
    if (!mul_ok((size_t)N, (size_t)(K / 32) * block_bytes, &w_want) || w_bytes != w_want)
        return Q4_ERR_SIZE;
    if (!mul_ok((size_t)M, (size_t)N, &y_bytes) || !mul_ok(y_bytes, sizeof(float), &y_bytes))
        return Q4_ERR_SIZE;
    if (M == 0 || N == 0) {
        *empty = true;
        return Q4_OK;
    }
    if (!gemv_streams(M, N, K, block_bytes, 4))
        return Q4_ERR_SHAPE;   // weight offsets beyond 31 bits
    const size_t need = gemv_prepare_bytes(M, K);
    if (prep_bytes < need)
        return Q4_ERR_SIZE;
    if (!prep || !w || !y)
        return Q4_ERR_NULL;
    if (!aligned16(prep) || !aligned16(w) || !aligned16(y))
        return Q4_ERR_ALIGN;
    if (overlaps({y, y_bytes}, {prep, need}) || overlaps({y, y_bytes}, {w, w_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

size_t gemv_splitk_workspace_bytes(int M, int N, int K, int requested, size_t block_bytes)
{
    if (M <= 0 || M > Q4_GEMV_MAX_ROWS || N <= 0 || K < 32 || K % 32 != 0 || requested < 0)
        return 0;
    const GemvSplit sp = gemv_split_plan(M, N, K, requested, block_bytes);
    if (sp.splits <= 1)
        return 0;
    size_t n = 0;
    if (!mul_ok((size_t)sp.splits * (size_t)M, (size_t)N, &n) || !mul_ok(n, 4, &n))
        return SIZE_MAX;
    return n;
}

size_t gemm_bf16_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K < 32 || K % 32 != 0)
        return 0;
    size_t n = 0;
    if (gemm_bf16_splits(M, N, K)) {
        // Rows padded to whole 128-row tiles, one binary16 per element.
        const size_t mp = ((size_t)M + 127) / 128 * 128;
        if (!mul_ok(mp, (size_t)K, &n) || !mul_ok(n, 2, &n))
            return SIZE_MAX;
    } else if (!mul_ok((size_t)M, (size_t)K, &n) || !mul_ok(n, 4, &n)) {
        return SIZE_MAX;
    }
    const size_t r = gemm_row_exp_bytes(M);
    return n > SIZE_MAX - r ? SIZE_MAX : n + r;
}

size_t gemm_q8a_workspace_bytes(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K < 32 || K % 32 != 0)
        return 0;
    size_t n = 0;
    if (gemm_splits_activations(K) && (long long)M * N < (1LL << 31)) {
        // Rows padded to whole 128-row tiles, two binary16 terms per element.
        const size_t mp = ((size_t)M + 127) / 128 * 128;
        if (!mul_ok(mp, (size_t)K, &n) || !mul_ok(n, 4, &n))
            return SIZE_MAX;
    } else if (!mul_ok((size_t)M, (size_t)K, &n) || !mul_ok(n, 4, &n)) {
        return SIZE_MAX;
    }
    const size_t r = gemm_row_exp_bytes(M);
    return n > SIZE_MAX - r ? SIZE_MAX : n + r;
}

int check_workspace(size_t need, const void *a, size_t a_elem, const void *w, size_t w_bytes,
                    const float *y, int M, int N, int K, const void *ws, size_t ws_bytes)
{
    return check_workspace_span(need, a, (size_t)M * (size_t)K * a_elem, w, w_bytes, y, M, N, ws,
                                ws_bytes);
}

int check_workspace_span(size_t need, const void *a, size_t a_bytes, const void *w, size_t w_bytes,
                         const float *y, int M, int N, const void *ws, size_t ws_bytes)
{
    if (need == 0)
        return Q4_OK;   // this shape takes no workspace; ws is not read
    if (need == SIZE_MAX)
        return Q4_ERR_SIZE;
    if (ws_bytes < need)
        return Q4_ERR_WORKSPACE;
    if (!ws)
        return Q4_ERR_NULL;
    if (!aligned16(ws))
        return Q4_ERR_ALIGN;
    const size_t y_bytes = (size_t)M * (size_t)N * sizeof(float);
    if (overlaps({ws, need}, {a, a_bytes}) || overlaps({ws, need}, {w, w_bytes}) ||
        overlaps({ws, need}, {y, y_bytes}))
        return Q4_ERR_ALIAS;
    return Q4_OK;
}

}  // namespace q4v
