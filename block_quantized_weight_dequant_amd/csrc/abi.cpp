// The exported C ABI (include/q4.h): validate every argument, then enqueue the
// kernel on the caller's stream. Only the functions declared in q4.h are
// exported from the shared library (it is built with hidden visibility).
#include "q4.h"

#include "launch.h"
#include "validate.h"

#define Q4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

int launched(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_LAUNCH; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

Q4_EXPORT int q4_abi_version(void) { return Q4_ABI_VERSION; }

Q4_EXPORT const char *q4_status_string(int status)
{
    switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "invalid shape (K must be a positive multiple of 32, sizes non-negative, "
                              "element counts a multiple of 32, GEMV rows in [0, 8])";
    case Q4_ERR_SIZE: return "a byte or element count does not match the shape";
    case Q4_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case Q4_ERR_ALIAS: return "an output overlaps an input";
    case Q4_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case Q4_ERR_WORKSPACE: return "the workspace is smaller than the GEMM's workspace_bytes function asks";
    default: return "unknown status";
    }
}

// Shared bodies of the Q4_0 and Q8_0 entry points.
static int dequant(q4k::WeightFormat fmt, size_t block_bytes, const void *w_q, size_t w_bytes,
                   float *out, size_t out_elems, void *stream)
{
    bool empty = false;
    int st = q4v::check_dequant(w_q, w_bytes, out, out_elems, block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_dequant(fmt, static_cast<const uint8_t *>(w_q), w_bytes / block_bytes,
                                        out, as_stream(stream)));
}

static int gemv(q4k::WeightFormat fmt, size_t block_bytes, const float *a, const void *w_q,
                size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, sizeof(float), w_q, w_bytes, y, M, N, K, Q4_GEMV_MAX_ROWS,
                                block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemv(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                     as_stream(stream)));
}

static int gemm(q4k::WeightFormat fmt, size_t block_bytes, const float *a, const void *w_q,
                size_t w_bytes, float *y, int M, int N, int K, void *workspace,
                size_t workspace_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, sizeof(float), w_q, w_bytes, y, M, N, K, 0, block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    st = q4v::check_workspace(q4v::gemm_workspace_bytes(M, N, K), a, sizeof(float), w_q, w_bytes,
                              y, M, N, K, workspace, workspace_bytes);
    if (st != Q4_OK)
        return st;
    return launched(q4k::launch_gemm(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                     workspace, as_stream(stream)));
}

static int gemm_noalloc(q4k::WeightFormat fmt, size_t block_bytes, const float *a, const void *w_q,
                        size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, sizeof(float), w_q, w_bytes, y, M, N, K, 0, block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemm_noalloc(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                             as_stream(stream)));
}

static int gemv_splitk(q4k::WeightFormat fmt, size_t block_bytes, const float *a, const void *w_q,
                       size_t w_bytes, float *y, int M, int N, int K, int splits, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, sizeof(float), w_q, w_bytes, y, M, N, K, Q4_GEMV_MAX_ROWS,
                                block_bytes, &empty);
    if (st != Q4_OK)
        return st;
    if (splits < 0)
        return Q4_ERR_SHAPE;
    if (empty)
        return Q4_OK;
    st = q4v::check_workspace(q4v::gemv_splitk_workspace_bytes(M, N, K, splits, block_bytes), a,
                              sizeof(float), w_q, w_bytes, y, M, N, K, workspace, workspace_bytes);
    if (st != Q4_OK)
        return st;
    return launched(q4k::launch_gemv_splitk(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                            q4v::gemv_split_plan(M, N, K, splits, block_bytes),
                                            workspace, as_stream(stream)));
}

static int gemv_prepare(q4k::WeightFormat fmt, const float *a, int M, int K, void *prep,
                        size_t prep_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_gemv_prepare(a, M, K, prep, prep_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemv_prepare(fmt, a, prep, M, K, as_stream(stream)));
}

static int gemv_prepared(q4k::WeightFormat fmt, size_t block_bytes, const void *prep,
                         size_t prep_bytes, const void *w_q, size_t w_bytes, float *y, int M,
                         int N, int K, void *stream)
{
    bool empty = false;
    int st = q4v::check_gemv_prepared(prep, prep_bytes, w_q, w_bytes, y, M, N, K, block_bytes,
                                      &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemv_prepared(fmt, prep, static_cast<const uint8_t *>(w_q), y, M,
                                              N, K, as_stream(stream)));
}

static int gemv_bf16(q4k::WeightFormat fmt, size_t block_bytes, const uint16_t *a,
                     const void *w_q, size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, 2, w_q, w_bytes, y, M, N, K, Q4_GEMV_MAX_ROWS, block_bytes,
                                &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemv_bf16(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                          as_stream(stream)));
}

static int gemv_q8a(q4k::WeightFormat fmt, size_t block_bytes, const void *a_q, size_t a_bytes,
                    const void *w_q, size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    bool empty = false;
    int st = q4v::check_product_q8a(a_q, a_bytes, w_q, w_bytes, y, M, N, K, Q4_GEMV_MAX_ROWS,
                                    block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_gemv_q8a(fmt, static_cast<const uint8_t *>(a_q),
                                         static_cast<const uint8_t *>(w_q), y, M, N, K,
                                         as_stream(stream)));
}

static int gemm_q8a(q4k::WeightFormat fmt, size_t block_bytes, const void *a_q, size_t a_bytes,
                    const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_product_q8a(a_q, a_bytes, w_q, w_bytes, y, M, N, K, 0, block_bytes,
                                    &empty);
    if (st != Q4_OK || empty)
        return st;
    st = q4v::check_workspace_span(q4v::gemm_q8a_workspace_bytes(M, N, K), a_q, a_bytes, w_q,
                                   w_bytes, y, M, N, workspace, workspace_bytes);
    if (st != Q4_OK)
        return st;
    return launched(q4k::launch_gemm_q8a(fmt, static_cast<const uint8_t *>(a_q),
                                         static_cast<const uint8_t *>(w_q), y, M, N, K, workspace,
                                         as_stream(stream)));
}

static int gemm_bf16(q4k::WeightFormat fmt, size_t block_bytes, const uint16_t *a,
                     const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_product(a, 2, w_q, w_bytes, y, M, N, K, 0, block_bytes, &empty);
    if (st != Q4_OK || empty)
        return st;
    st = q4v::check_workspace(q4v::gemm_bf16_workspace_bytes(M, N, K), a, 2, w_q, w_bytes, y, M,
                              N, K, workspace, workspace_bytes);
    if (st != Q4_OK)
        return st;
    return launched(q4k::launch_gemm_bf16(fmt, a, static_cast<const uint8_t *>(w_q), y, M, N, K,
                                          workspace, as_stream(stream)));
}

Q4_EXPORT int q4_dequant(const void *w_q, size_t w_bytes, float *out, size_t out_elems, void *stream)
{
    return dequant(q4k::WeightFormat::kQ4_0, 18, w_q, w_bytes, out, out_elems, stream);
}

Q4_EXPORT int q8_dequant(const void *w_q, size_t w_bytes, float *out, size_t out_elems, void *stream)
{
    return dequant(q4k::WeightFormat::kQ8_0, 34, w_q, w_bytes, out, out_elems, stream);
}

Q4_EXPORT int q4_gemv(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                      void *stream)
{
    return gemv(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT int q8_gemv(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                      void *stream)
{
    return gemv(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT size_t q4_gemm_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_workspace_bytes(M, N, K);
}

Q4_EXPORT size_t q8_gemm_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_workspace_bytes(M, N, K);
}

Q4_EXPORT int q4_gemm(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                      void *stream)
{
    return gemm_noalloc(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT int q8_gemm(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N, int K,
                      void *stream)
{
    return gemm_noalloc(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT int q4_gemm_ws(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N,
                         int K, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, workspace,
                workspace_bytes, stream);
}

Q4_EXPORT int q8_gemm_ws(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N,
                         int K, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, workspace,
                workspace_bytes, stream);
}

Q4_EXPORT int q4_gemv_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y, int M,
                           int N, int K, void *stream)
{
    return gemv_bf16(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT int q8_gemv_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y, int M,
                           int N, int K, void *stream)
{
    return gemv_bf16(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT size_t q4_gemv_prepare_bytes(int M, int K) { return q4v::gemv_prepare_bytes(M, K); }

Q4_EXPORT size_t q8_gemv_prepare_bytes(int M, int K) { return q4v::gemv_prepare_bytes(M, K); }

Q4_EXPORT int q4_gemv_prepare(const float *a, int M, int K, void *prep, size_t prep_bytes,
                              void *stream)
{
    return gemv_prepare(q4k::WeightFormat::kQ4_0, a, M, K, prep, prep_bytes, stream);
}

Q4_EXPORT int q8_gemv_prepare(const float *a, int M, int K, void *prep, size_t prep_bytes,
                              void *stream)
{
    return gemv_prepare(q4k::WeightFormat::kQ8_0, a, M, K, prep, prep_bytes, stream);
}

Q4_EXPORT int q4_gemv_prepared(const void *prep, size_t prep_bytes, const void *w_q,
                               size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    return gemv_prepared(q4k::WeightFormat::kQ4_0, 18, prep, prep_bytes, w_q, w_bytes, y, M, N, K,
                         stream);
}

Q4_EXPORT int q8_gemv_prepared(const void *prep, size_t prep_bytes, const void *w_q,
                               size_t w_bytes, float *y, int M, int N, int K, void *stream)
{
    return gemv_prepared(q4k::WeightFormat::kQ8_0, 34, prep, prep_bytes, w_q, w_bytes, y, M, N, K,
                         stream);
}

Q4_EXPORT size_t q4_gemv_splitk_workspace_bytes(int M, int N, int K, int splits)
{
    return q4v::gemv_splitk_workspace_bytes(M, N, K, splits, 18);
}

Q4_EXPORT size_t q8_gemv_splitk_workspace_bytes(int M, int N, int K, int splits)
{
    return q4v::gemv_splitk_workspace_bytes(M, N, K, splits, 34);
}

Q4_EXPORT int q4_gemv_splitk(const float *a, const void *w_q, size_t w_bytes, float *y, int M,
                             int N, int K, int splits, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    return gemv_splitk(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, splits,
                       workspace, workspace_bytes, stream);
}

Q4_EXPORT int q8_gemv_splitk(const float *a, const void *w_q, size_t w_bytes, float *y, int M,
                             int N, int K, int splits, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    return gemv_splitk(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, splits,
                       workspace, workspace_bytes, stream);
}

Q4_EXPORT size_t q4_gemm_bf16_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_bf16_workspace_bytes(M, N, K);
}

Q4_EXPORT size_t q8_gemm_bf16_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_bf16_workspace_bytes(M, N, K);
}

Q4_EXPORT int q4_gemm_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y, int M,
                           int N, int K, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_bf16(q4k::WeightFormat::kQ4_0, 18, a, w_q, w_bytes, y, M, N, K, workspace,
                     workspace_bytes, stream);
}

Q4_EXPORT int q8_gemm_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y, int M,
                           int N, int K, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_bf16(q4k::WeightFormat::kQ8_0, 34, a, w_q, w_bytes, y, M, N, K, workspace,
                     workspace_bytes, stream);
}

Q4_EXPORT int q8_quantize(const float *x, size_t n_elems, void *out_q, size_t out_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_quantize(x, n_elems, out_q, out_bytes, 34, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_q8_quantize(x, n_elems / 32, static_cast<uint8_t *>(out_q),
                                            as_stream(stream)));
}

Q4_EXPORT int q4_quantize(const float *x, size_t n_elems, void *out_q, size_t out_bytes, void *stream)
{
    bool empty = false;
    int st = q4v::check_quantize(x, n_elems, out_q, out_bytes, 18, &empty);
    if (st != Q4_OK || empty)
        return st;
    return launched(q4k::launch_q4_quantize(x, n_elems / 32, static_cast<uint8_t *>(out_q),
                                            as_stream(stream)));
}

Q4_EXPORT int q4_gemv_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes,
                          float *y, int M, int N, int K, void *stream)
{
    return gemv_q8a(q4k::WeightFormat::kQ4_0, 18, a_q, a_bytes, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT int q8_gemv_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes,
                          float *y, int M, int N, int K, void *stream)
{
    return gemv_q8a(q4k::WeightFormat::kQ8_0, 34, a_q, a_bytes, w_q, w_bytes, y, M, N, K, stream);
}

Q4_EXPORT size_t q4_gemm_q8a_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_q8a_workspace_bytes(M, N, K);
}

Q4_EXPORT size_t q8_gemm_q8a_workspace_bytes(int M, int N, int K)
{
    return q4v::gemm_q8a_workspace_bytes(M, N, K);
}

Q4_EXPORT int q4_gemm_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes,
                          float *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
                          void *stream)
{
    return gemm_q8a(q4k::WeightFormat::kQ4_0, 18, a_q, a_bytes, w_q, w_bytes, y, M, N, K,
                    workspace, workspace_bytes, stream);
}

Q4_EXPORT int q8_gemm_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes,
                          float *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
                          void *stream)
{
    return gemm_q8a(q4k::WeightFormat::kQ8_0, 34, a_q, a_bytes, w_q, w_bytes, y, M, N, K,
                    workspace, workspace_bytes, stream);
}
