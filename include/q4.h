/*
 * q4.h — C ABI of the MI355X (gfx950) block-quantized (GGML Q4_0 / Q8_0)
 * weight library.
 *
 * Formats (docs.rs fuel-dispatch 0.20.71, page "fuel-vulkan-kernels — quantized
 * (GGML) kernel contracts"):
 *   Q4_0 block (section dequant_q4_0): 18 bytes for 32 elements, a little-endian
 *     binary16 scale d, then 16 bytes; the low nibble of byte j is element j and
 *     the high nibble is element j+16; element = (nibble - 8) * d, d widened to f32.
 *   Q8_0 block (sections dequant_q8_0, quantize_q8_0): 34 bytes for 32 elements,
 *     a little-endian binary16 scale d, then 32 signed bytes; element = q * d.
 *   Weight matrix W[N, K/32] (sections qmatvec_q4_0, matmul_q4_0_tiled): a
 *     contiguous row-major block stream, K/32 blocks per row, N * (K/32) * 18
 *     bytes in all for Q4_0 and N * (K/32) * 34 for Q8_0, read from its first
 *     byte (no strides, no offsets). The quantized-matmul binding on the page
 *     picks Q4_0 or Q8_0 blocks by quant type; the q8_* products are the q4_*
 *     ones over Q8_0 weights.
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller; the library
 *     allocates and frees nothing and keeps no state between calls, except
 *     the device scratch of q4_gemm and q8_gemm (below), whose contents no
 *     call relies on.
 *   - Every pointer must be 16-byte aligned (the pages' alignment_bytes: 16),
 *     else Q4_ERR_ALIGN. Arrays are dense and contiguous; f32 matrices are
 *     row-major.
 *   - Outputs are fully overwritten, never accumulated into, and must not
 *     overlap any input (the pages: aliasing none, in_place false), else
 *     Q4_ERR_ALIAS. No byte outside an output's stated extent is written.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls are asynchronous: arguments are checked, the work is enqueued on
 *     `stream`, and the call returns without synchronizing.
 *   - Every argument error is detected before anything is launched, and then
 *     nothing is written. Device faults surface at the caller's next
 *     synchronization. An empty problem (a zero dimension or element count)
 *     returns Q4_OK and launches nothing; its pointers may be NULL.
 *   - Inputs are finite; results for NaN or infinite inputs are unspecified.
 */
#ifndef Q4MI_Q4_H
#define Q4MI_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 10

#define Q4_OK 0
#define Q4_ERR_NULL 1   /* a required pointer is NULL */
#define Q4_ERR_SHAPE 2  /* K % 32 != 0, K < 32, a negative size, M outside the GEMV range, n % 32 != 0 */
#define Q4_ERR_SIZE 3   /* a byte or element count disagrees with the shape, or overflows size_t */
#define Q4_ERR_ALIGN 4  /* a pointer is not 16-byte aligned */
#define Q4_ERR_ALIAS 5  /* an output overlaps an input */
#define Q4_ERR_LAUNCH 6 /* the HIP runtime refused the launch */
#define Q4_ERR_WORKSPACE 7 /* a GEMM workspace is smaller than its *_gemm_workspace_bytes */

/* Largest number of activation rows q4_gemv and q8_gemv accept. */
#define Q4_GEMV_MAX_ROWS 8

/* Bytes of device memory each GPU holds for q4_gemm and q8_gemm (64 MiB). */
#define Q4_GEMM_SCRATCH_BYTES 67108864u

/* Returns Q4_ABI_VERSION of the library actually loaded. */
int q4_abi_version(void);

/* Returns a static, NUL-terminated description of a status code. */
const char *q4_status_string(int status);

/*
 * q4_dequant — Q4_0 block stream to dense f32 (section dequant_q4_0).
 *   w_q       n_blocks * 18 bytes of Q4_0 blocks, with n_blocks = w_bytes / 18.
 *   w_bytes   must be a multiple of 18 (else Q4_ERR_SIZE).
 *   out       out_elems f32; out_elems must equal w_bytes / 18 * 32 (else
 *             Q4_ERR_SIZE). Element 32*b + j of out is element j of block b.
 * Bit-exact: every output is the exact product (nibble - 8) * d, so results
 * equal any correct evaluation bit for bit, signed zeros included.
 */
int q4_dequant(const void *w_q, size_t w_bytes, float *out, size_t out_elems, void *stream);

/*
 * q4_gemv — decode-shaped product y = a @ dequant(W)^T for 1 <= M <= 8
 * activation rows (section qmatvec_q4_0, widened from one row to eight).
 *   a         [M, K] f32, row-major.
 *   w_q       W[N, K/32] Q4_0 block stream; w_bytes == N * (K/32) * 18.
 *   y         [M, N] f32, row-major: y[m, n] = sum_k a[m, k] * w[n, k].
 *   M in [1, 8], N >= 1, K >= 32 and K % 32 == 0 (else Q4_ERR_SHAPE);
 *   M == 0 or N == 0 is an empty problem.
 * Accuracy: |y - y_exact| <= 1e-5 * sum_k |a[m, k] * w[n, k]| + 1e-6 per
 * element. Each stretch of K that the kernel handles at once is scaled by
 * the power of two that puts its largest A value in [2^14, 2^15) and split
 * into two binary16 terms; binary16's floor adds a second term: each
 * activation's split is within 2^-22 of it or within 2^-35 (2^-39 for
 * q8_gemv) of its row's largest magnitude, whichever is larger, so a row
 * whose magnitudes span more than about 2^18 can add up to
 * 2^-35 * max|a[m, :]| * sum_k |w[n, k]|. The reduction order is fixed, so
 * repeated calls return identical bits.
 * Speed: with w_q 128-byte aligned and K % 2048 == 0 every weight row is a
 * whole number of cache lines and is fetched in whole lines (about 2-9%
 * faster); other 16-byte aligned streams give the same bits.
 */
int q4_gemv(const float *a, const void *w_q, size_t w_bytes, float *y,
            int M, int N, int K, void *stream);

/*
 * q4_gemm — the prefill GEMM of q4_gemm_ws with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The operation is
 * section matmul_q4_0_tiled's, y = a @ dequant(W)^T for any M >= 1.
 *   a, w_q, w_bytes, y, M, N, K, stream: as q4_gemm_ws; errors as q4_gemm_ws's
 *             checks before its workspace; no size is rejected.
 * Scratch: the library's own device array of Q4_GEMM_SCRATCH_BYTES, held by
 * each GPU the library runs on until the process ends (its address is looked
 * up on the first call on a device). The call allocates and frees nothing.
 * Rows are taken in chunks whose row exponents and operands fit the array
 * (whole 128-row tiles; 16384 rows at K = 4096), one after another on
 * `stream`, so the results equal q4_gemm_ws's bit for bit; for K >= 131072 a
 * tile's operands do not fit and the general kernel runs (the accuracy bound
 * of q4_gemm_ws's general-kernel shapes). Calls that overlap in time on one
 * GPU (on different streams, or from different threads) share the array and
 * race: the caller orders them, or uses q4_gemm_ws with its own workspaces.
 * Accuracy and determinism as q4_gemm_ws.
 */
int q4_gemm(const float *a, const void *w_q, size_t w_bytes, float *y,
            int M, int N, int K, void *stream);

/* q8_gemm — q4_gemm over a Q8_0 weight stream (w_bytes == N * (K/32) * 34),
 * for the same callers; it shares q4_gemm's scratch array (and its race). */
int q8_gemm(const float *a, const void *w_q, size_t w_bytes, float *y,
            int M, int N, int K, void *stream);

/*
 * q4_gemm_ws — prefill-shaped product y = a @ dequant(W)^T for any M >= 1
 * (section matmul_q4_0_tiled), tiled through LDS onto the matrix cores, with
 * the caller's scratch memory.
 *   a, w_q, w_bytes, y, M, N, K: as q4_gemv, with M >= 1 unbounded (M == 0 or
 *             N == 0 is an empty problem). Any finite activations: each row
 *             of a is scaled by the power of two that puts its largest
 *             magnitude in [2^14, 2^15), split into two binary16 terms
 *             (within 2^-22 of each scaled element) and the result row is
 *             scaled back.
 *   workspace, workspace_bytes: device scratch owned by the caller, at least
 *             q4_gemm_workspace_bytes(M, N, K) bytes (non-zero for every
 *             non-empty shape), 16-byte aligned, not overlapping a, W or y,
 *             and not used by other work while this call runs on `stream`.
 *             Errors, after those of q4_gemv's checks: Q4_ERR_SIZE if the
 *             needed size overflows size_t, Q4_ERR_WORKSPACE if
 *             workspace_bytes is smaller, then Q4_ERR_NULL, Q4_ERR_ALIGN,
 *             Q4_ERR_ALIAS for the pointer. The library allocates nothing,
 *             so the call may be captured in a HIP graph; the workspace's
 *             contents after the call are unspecified.
 * Accuracy: |y - y_exact| <= 1e-5 * sum_k |a[m, k] * w[n, k]| + 1e-6 per
 * element. The worst-case error is (36 + L + S) * 2^-24 of that sum, to first
 * order: 4 for the split, 32 for a block's 32 products, L <= 112 block
 * partials added in sequence per accumulator, and S K segments (longer K runs
 * as several launches, each adding its part to y); S = ceil(K / 7168) when
 * K % 64 == 0, K <= 2^22 and M * N < 2^31, else ceil(K / 3584) (one fewer
 * term). This stays below 1e-5 for K <= 136192 (K <= 71680 on the other
 * shapes). Binary16's floor adds a second term: each activation's split is
 * within 2^-22 of it or within 2^-46 of its row's largest magnitude,
 * whichever is larger, so a row whose magnitudes span more than 2^24 can add
 * up to 2^-46 * max|a[m, :]| * sum_k |w[n, k]|. The reduction order is
 * fixed, so repeated calls return identical bits.
 */
int q4_gemm_ws(const float *a, const void *w_q, size_t w_bytes, float *y,
               int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_gemm_workspace_bytes — bytes of workspace q4_gemm_ws needs for this
 * shape: the row exponents (M int32, padded to a multiple of 256 bytes), then,
 * when K % 64 == 0, K <= 2^22 and M * N < 2^31, ceil(M / 128) * 128 * K * 4
 * bytes of operands (the scaled activations split once into binary16 hi and
 * lo terms, in matrix-core operand order). 0 when M, N or K is invalid or the
 * problem is empty, and SIZE_MAX when the size does not fit in size_t. Pure
 * function of its arguments.
 */
size_t q4_gemm_workspace_bytes(int M, int N, int K);

/*
 * q8_dequant — Q8_0 block stream to dense f32 (section dequant_q8_0).
 *   w_q       n_blocks * 34 bytes of Q8_0 blocks, with n_blocks = w_bytes / 34.
 *   w_bytes   must be a multiple of 34 (else Q4_ERR_SIZE).
 *   out       out_elems f32; out_elems must equal w_bytes / 34 * 32 (else
 *             Q4_ERR_SIZE). Element 32*b + j of out is element j of block b.
 * Bit-exact: every output is the exact product q * d (q the signed byte), so
 * results equal any correct evaluation bit for bit, signed zeros included.
 */
int q8_dequant(const void *w_q, size_t w_bytes, float *out, size_t out_elems, void *stream);

/*
 * q8_gemv — q4_gemv over a Q8_0 weight stream: y = a @ dequant(W)^T for
 * 1 <= M <= 8, with w_bytes == N * (K/32) * 34. Arguments, errors, accuracy
 * and determinism as q4_gemv.
 */
int q8_gemv(const float *a, const void *w_q, size_t w_bytes, float *y,
            int M, int N, int K, void *stream);

/*
 * q8_gemm_ws — q4_gemm_ws over a Q8_0 weight stream, with w_bytes == N * (K/32)
 * * 34. Arguments, errors, accuracy, the workspace contract (with
 * q8_gemm_workspace_bytes) and determinism as q4_gemm_ws.
 */
int q8_gemm_ws(const float *a, const void *w_q, size_t w_bytes, float *y,
               int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/*
 * q8_gemm_workspace_bytes — bytes of workspace q8_gemm_ws needs for this
 * shape; the same function of (M, N, K) as q4_gemm_workspace_bytes.
 */
size_t q8_gemm_workspace_bytes(int M, int N, int K);

/*
 * q4_gemv_prepare / q4_gemv_prepared — the decode GEMV in two steps, for
 * activations that several weight matrices multiply (the projections that
 * share one input) and for M > 1, where every workgroup of q4_gemv splits the
 * same f32 activations into matrix-core operands (section qmatvec_q4_0,
 * widened to eight rows as q4_gemv).
 *   q4_gemv_prepare(a, M, K, prep, prep_bytes, stream): a [M, K] f32,
 *     1 <= M <= 8, K a positive multiple of 256 (else Q4_ERR_SHAPE); writes
 *     q4_gemv_prepare_bytes(M, K) bytes of prepared operands to prep
 *     (prep_bytes smaller: Q4_ERR_SIZE). Each row is scaled by the power of
 *     two that puts its largest magnitude (times 16, the Q4_0 decode's factor)
 *     in [2^14, 2^15), then split into two binary16 terms per element in
 *     matrix-core operand order; the row exponents follow. M == 0 is empty.
 *   q4_gemv_prepared(prep, prep_bytes, w_q, w_bytes, y, M, N, K, stream):
 *     y = a @ dequant(W)^T from prep (made by q4_gemv_prepare for the same M
 *     and K), w_q and y as q4_gemv. Shape errors as q4_gemv_prepare, and
 *     Q4_ERR_SHAPE when W exceeds 2^31 bytes; sizes, pointers and overlap as
 *     q4_gemv, with prep in place of a.
 * The prepared buffer is specific to the weight format (q8_gemv_prepare's
 * differs). Accuracy as q4_gemv (the floor relative to the whole row's
 * largest magnitude); deterministic. Measured on MI355X (N = K = 4096, cold
 * weights), the prepared GEMV is faster than q4_gemv from M = 3 up (8 rows:
 * 5.4 us against 6.2 us, plus 3.1 us to prepare, once per shared input) and
 * q8_gemv_prepared than q8_gemv from M = 5 up; with fewer rows the one-step
 * GEMV is faster (one row: 4.25 against 5.1 us).
 */
size_t q4_gemv_prepare_bytes(int M, int K);
int q4_gemv_prepare(const float *a, int M, int K, void *prep, size_t prep_bytes, void *stream);
int q4_gemv_prepared(const void *prep, size_t prep_bytes, const void *w_q, size_t w_bytes,
                     float *y, int M, int N, int K, void *stream);

/* q8_gemv_prepare / q8_gemv_prepared — the same two steps for Q8_0 weights
 * (the row scale puts the largest magnitude itself in [2^14, 2^15)). */
size_t q8_gemv_prepare_bytes(int M, int K);
int q8_gemv_prepare(const float *a, int M, int K, void *prep, size_t prep_bytes, void *stream);
int q8_gemv_prepared(const void *prep, size_t prep_bytes, const void *w_q, size_t w_bytes,
                     float *y, int M, int N, int K, void *stream);

/*
 * q4_gemv_splitk — q4_gemv with K split across workgroups, for decode shapes
 * with few output columns per compute unit (for example one GPU's share of a
 * weight split by rows) and long rows. Splitting the reduction over K is the
 * direction of virtio-accel ADR 10 ("Vulkan kernel throughput ...", section
 * Consequences) for a GEMV whose flat geometry stalls.
 *   a, w_q, w_bytes, y, M, N, K: as q4_gemv (1 <= M <= 8).
 *   splits    0 lets the library choose: no split when the plain GEMV
 *             walks fewer than 3 chunks of K per wavefront (K < 12288 or so),
 *             else enough workgroups for 256 compute units, ceil(256 /
 *             ceil(N / 16)), at most one per 64 blocks of K. A positive value
 *             asks for that many. Either is capped at one
 *             split per 8 blocks of K, and rounded so every split holds a
 *             multiple of 8 blocks (the last one the rest). Negative:
 *             Q4_ERR_SHAPE.
 *   workspace, workspace_bytes: at least q4_gemv_splitk_workspace_bytes(M,
 *             N, K, splits) bytes of device scratch (the splits' partial
 *             outputs), as for q4_gemm; 0 bytes (NULL allowed) when the call
 *             does not split: one split, or K % 256 != 0 (then it is q4_gemv).
 * Each split writes its partial y; a second kernel adds the partials in split
 * order, so repeated calls return identical bits. Accuracy: as q4_gemv.
 */
int q4_gemv_splitk(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N,
                   int K, int splits, void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_gemv_splitk_workspace_bytes — splits * M * N * 4 for the split the call
 * would use, 0 when it does not split or the shape is invalid or empty,
 * SIZE_MAX on overflow. Pure function of its arguments.
 */
size_t q4_gemv_splitk_workspace_bytes(int M, int N, int K, int splits);

/* q8_gemv_splitk — q4_gemv_splitk over a Q8_0 weight stream (w_bytes == N * (K/32) * 34). */
int q8_gemv_splitk(const float *a, const void *w_q, size_t w_bytes, float *y, int M, int N,
                   int K, int splits, void *workspace, size_t workspace_bytes, void *stream);

/* q8_gemv_splitk_workspace_bytes — as q4_gemv_splitk_workspace_bytes, for q8_gemv_splitk. */
size_t q8_gemv_splitk_workspace_bytes(int M, int N, int K, int splits);

/*
 * q4_gemv_bf16 — q4_gemv with bfloat16 activations: y = a @ dequant(W)^T for
 * 1 <= M <= 8, y in f32 (section qmatvec_q4_0 as for q4_gemv; the activation
 * type is the one of the 4-bit workload in TensorFold pull request #2017,
 * section Setup, whose own 4-bit format is another one).
 *   a         [M, K] bfloat16, row-major, as raw 16-bit patterns.
 *   w_q, y, M, N, K: as q4_gemv. Errors: as q4_gemv, with a counted at
 *             2 bytes per element.
 * The activations of each row are scaled, per stretch of K the kernel
 * handles at once (256 or 512 elements of K on 16-byte aligned rows, the whole
 * row otherwise), by a power of two that brings the stretch's largest
 * magnitude to [2^15, 2^16) on the matrix-core operand; every element within
 * 2^28 of that magnitude (2^32 for q8_gemv_bf16) is then an exact binary16
 * number and each product with a weight code is exact in f32. Smaller
 * elements are rounded to 2^-24 on the scaled grid. Accuracy, for rows within
 * that range: as q4_gemv. Deterministic.
 */
int q4_gemv_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y,
                 int M, int N, int K, void *stream);

/* q8_gemv_bf16 — q4_gemv_bf16 over a Q8_0 weight stream (w_bytes == N * (K/32) * 34). */
int q8_gemv_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y,
                 int M, int N, int K, void *stream);

/*
 * q4_gemm_bf16 — q4_gemm with bfloat16 activations: y = a @ dequant(W)^T for
 * any M >= 1, y in f32. The 4-bit prefill measured in TensorFold pull request
 * #2017 ("Vulkan: qmm_q4_tile_rows computes four rows and two columns of a
 * prompt chunk per thread", section Setup) multiplies bfloat16 activations;
 * that checkpoint's 4-bit format is another one, so only the activation type
 * is taken from it, and the weight blocks are those of section dequant_q4_0,
 * as for q4_gemm.
 *   a         [M, K] bfloat16, row-major, as raw 16-bit patterns (the high
 *             half of the f32 with the same value).
 *   w_q, y, M, N, K: as q4_gemm (w_bytes == N * (K/32) * 18).
 *   workspace, workspace_bytes: as q4_gemm's, sized by
 *             q4_gemm_bf16_workspace_bytes, which is non-zero for every
 *             non-empty shape (the workspace is always used).
 * Each row of a is scaled by a power of two 2^p that brings its largest
 * magnitude into [2^15, 2^16); every element within 2^28 of that magnitude
 * (2^32 for q8_gemm_bf16) is then exactly a binary16 number, the products
 * with the weight codes are exact in f32, and the row of y is scaled back by
 * 2^-p. Elements further below the row maximum are rounded to 2^-24 on the
 * scaled grid. Accuracy, for rows within that range: as q4_gemm. Errors: as
 * q4_gemm, with a counted at 2 bytes per element. Deterministic.
 */
int q4_gemm_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y,
                 int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_gemm_bf16_workspace_bytes — bytes of workspace q4_gemm_bf16 needs:
 * the row exponents (M int32, padded to a multiple of 256 bytes), then
 * ceil(M / 128) * 128 * K * 2 when K % 64 == 0, K <= 2^22 and M * N < 2^31 (one binary16
 * term per activation, in matrix-core operand order), else M * K * 4 (the
 * scaled activations in f32). 0 when M, N or K is invalid or the problem is
 * empty, SIZE_MAX when the size does not fit in size_t. Pure function.
 */
size_t q4_gemm_bf16_workspace_bytes(int M, int N, int K);

/*
 * q8_gemm_bf16 — q4_gemm_bf16 over a Q8_0 weight stream (w_bytes ==
 * N * (K/32) * 34); exact for elements within 2^32 of their row's largest
 * magnitude. Everything else as q4_gemm_bf16.
 */
int q8_gemm_bf16(const uint16_t *a, const void *w_q, size_t w_bytes, float *y,
                 int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/* q8_gemm_bf16_workspace_bytes — the same function as q4_gemm_bf16_workspace_bytes. */
size_t q8_gemm_bf16_workspace_bytes(int M, int N, int K);

/*
 * q4_gemv_q8a — the decode GEMV over activations quantized to Q8_0 blocks
 * along K. The geistlib issue "vulkan: shader and sequencing efficiency
 * backlog" names an activation-quantize kernel and its fusion without
 * defining them; here each activation row is a run of Q8_0 blocks as
 * q8_quantize writes them (section quantize_q8_0; any Q8_0 blocks are
 * accepted), and y = dequant_q8_0(a_q) @ dequant(W)^T, that is
 * y[m, n] = sum over blocks b of d_w[n, b] d_a[m, b] sum_j w_code q_a
 * (sections dequant_q8_0, dequant_q4_0 and qmatvec_q4_0).
 *   a_q       the [M, K/32] Q8_0 block stream of the activations, row m's
 *             blocks contiguous in K order; a_bytes == M * (K/32) * 34.
 *   w_q, w_bytes, y, M, N, K: as q4_gemv (1 <= M <= 8).
 * Errors as q4_gemv, with a_bytes checked like w_bytes (Q4_ERR_SIZE).
 * The block sums are integer and exact on the matrix cores; each is scaled by
 * d_w d_a (exact in f32) and added with one rounding. Accuracy: |y - y_exact|
 * <= 1e-5 * sum_k |a'[m, k] w[n, k]| + 1e-6, a' the dequantized activations.
 * Against the f32 activations the quantization itself adds up to
 * d_a / 2 per element. Deterministic.
 */
int q4_gemv_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes, float *y,
                int M, int N, int K, void *stream);

/* q8_gemv_q8a — q4_gemv_q8a over a Q8_0 weight stream (w_bytes == N * (K/32) * 34). */
int q8_gemv_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes, float *y,
                int M, int N, int K, void *stream);

/*
 * q4_gemm_q8a — the prefill product over Q8_0-quantized activations, any
 * M >= 1: y = dequant_q8_0(a_q) @ dequant(W)^T as q4_gemv_q8a (section
 * matmul_q4_0_tiled for the product; the activation blocks as there).
 *   a_q, a_bytes: the [M, K/32] Q8_0 block stream, a_bytes == M * (K/32) * 34.
 *   w_q, w_bytes, y, M, N, K: as q4_gemm.
 *   workspace, workspace_bytes: at least q4_gemm_q8a_workspace_bytes(M, N, K)
 *             bytes of device scratch, 16-byte aligned, overlapping nothing
 *             else (smaller: Q4_ERR_WORKSPACE); always used for M, N > 0.
 * Each dequantized activation (an 8-bit code times a binary16 scale) is exact
 * in f32; every row is scaled by the power of two that puts 128 times its
 * largest |d| in [2^14, 2^15) and split into two binary16 terms, then
 * multiplied as in q4_gemm and scaled back. The two terms hold every
 * dequantized activation exactly (its last bit never falls below the lo
 * term's grid), with one exception in q4_gemm_q8a, whose high-nibble slots
 * take a / 16: on a row whose largest |d| is 2^15 or more, activations of
 * blocks with |d| below 2^-13 are rounded to within 2^-24 (2^-39 of that
 * largest |d|). Accuracy: as q4_gemv_q8a, plus that rounding on such rows.
 * Deterministic. Errors: as q4_gemm, with a_bytes checked like w_bytes.
 */
int q4_gemm_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes, float *y,
                int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/* q4_gemm_q8a_workspace_bytes — the row exponents (M int32, padded to 256
 * bytes), then ceil(M/128) * 128 * K * 4 bytes of operands when K % 64 == 0,
 * K <= 2^22 and M * N < 2^31, else M * K * 4; 0 for an empty or invalid shape,
 * SIZE_MAX when it does not fit in size_t. */
size_t q4_gemm_q8a_workspace_bytes(int M, int N, int K);

/* q8_gemm_q8a — q4_gemm_q8a over a Q8_0 weight stream; the same workspace. */
int q8_gemm_q8a(const void *a_q, size_t a_bytes, const void *w_q, size_t w_bytes, float *y,
                int M, int N, int K, void *workspace, size_t workspace_bytes, void *stream);

/* q8_gemm_q8a_workspace_bytes — the same function as q4_gemm_q8a_workspace_bytes. */
size_t q8_gemm_q8a_workspace_bytes(int M, int N, int K);

/*
 * q8_quantize — f32 to Q8_0 blocks (section quantize_q8_0).
 *   x         n_elems f32; n_elems % 32 == 0 (else Q4_ERR_SHAPE).
 *   out_q     out_bytes == n_elems / 32 * 34 (else Q4_ERR_SIZE).
 * Per 32-element block: d = max|x| / 127 in f32; the binary16 d (round to
 * nearest even) is stored little-endian, then 32 bytes q = round(x / d) in
 * two's complement, with round() half away from zero, the quotient formed from
 * the f32 d, and q = 0 (d = +0) for an all-zero block. Bit-exact and
 * deterministic.
 */
int q8_quantize(const float *x, size_t n_elems, void *out_q, size_t out_bytes, void *stream);

/*
 * q4_quantize — f32 to Q4_0 blocks with GGML's reference rule: per 32-element
 * block, d = (the element of largest |x|, the first on ties) / -8 in f32, the
 * binary16 d stored little-endian, then q_j = min(15, (int)(x_j / d + 8.5)) in
 * two separately rounded f32 operations (q = 8 throughout when d == 0), packed
 * as byte j = q_j | q_{j+16} << 4. This rule is not on the pages; it makes
 * Q4_0 weights on the device from f32 ones.
 *   x         n_elems f32; n_elems % 32 == 0 (else Q4_ERR_SHAPE).
 *   out_q     out_bytes == n_elems / 32 * 18 (else Q4_ERR_SIZE).
 * Bit-exact and deterministic.
 */
int q4_quantize(const float *x, size_t n_elems, void *out_q, size_t out_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4MI_Q4_H */
