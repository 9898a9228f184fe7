// Kernel launchers behind the C ABI. Each validates nothing (the ABI layer has
// already checked every argument) and returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q4.h"
#include "validate.h"

namespace q4k {

// Block format of a weight stream.
enum class WeightFormat { kQ4_0, kQ8_0 };

hipError_t launch_dequant(WeightFormat fmt, const uint8_t *w, size_t n_blocks, float *out,
                          hipStream_t s);
hipError_t launch_gemv(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M, int N,
                       int K, hipStream_t s);
// a: [M, K] bfloat16 bit patterns, 1 <= M <= 8.
hipError_t launch_gemv_bf16(WeightFormat fmt, const uint16_t *a, const uint8_t *w, float *y, int M,
                            int N, int K, hipStream_t s);
// Prepared activations for the GEMV: launch_gemv_prepare writes
// q4v::gemv_prepare_bytes(M, K) bytes of operands for the format; the
// prepared GEMV reads them instead of `a` (K % 256 == 0 only).
hipError_t launch_gemv_prepare(WeightFormat fmt, const float *a, void *prep, int M, int K,
                               hipStream_t s);
hipError_t launch_gemv_prepared(WeightFormat fmt, const void *prep, const uint8_t *w, float *y,
                                int M, int N, int K, hipStream_t s);
// a_q: the [M, K/32] Q8_0 block stream of the activations, 1 <= M <= 8.
hipError_t launch_gemv_q8a(WeightFormat fmt, const uint8_t *a_q, const uint8_t *w, float *y, int M,
                           int N, int K, hipStream_t s);
// K split across workgroups: partials of sp.splits splits into `workspace`
// (sp.splits * M * N f32), then summed into y in split order. sp.splits <= 1
// runs launch_gemv's kernel (workspace unused).
hipError_t launch_gemv_splitk(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M,
                              int N, int K, const q4v::GemvSplit &sp, void *workspace,
                              hipStream_t s);
// workspace: q4v::gemm_workspace_bytes(M, N, K) bytes (always used: the row
// exponents, then on the split path the two-term operands).
hipError_t launch_gemm(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M, int N,
                       int K, void *workspace, hipStream_t s);
// The same without a workspace: the library's own device scratch of
// kGemmScratchBytes per GPU, rows taken in chunks that fit it. Calls that
// overlap in time on one GPU race on the scratch.
constexpr size_t kGemmScratchBytes = Q4_GEMM_SCRATCH_BYTES;
hipError_t launch_gemm_noalloc(WeightFormat fmt, const float *a, const uint8_t *w, float *y, int M,
                               int N, int K, hipStream_t s);
// a: [M, K] bfloat16 bit patterns. workspace:
// q4v::gemm_bf16_workspace_bytes(M, N, K) bytes (always used).
hipError_t launch_gemm_bf16(WeightFormat fmt, const uint16_t *a, const uint8_t *w, float *y, int M,
                            int N, int K, void *workspace, hipStream_t s);
// a_q: the [M, K/32] Q8_0 block stream of the activations. workspace:
// q4v::gemm_q8a_workspace_bytes(M, N, K) bytes (always used).
hipError_t launch_gemm_q8a(WeightFormat fmt, const uint8_t *a_q, const uint8_t *w, float *y, int M,
                           int N, int K, void *workspace, hipStream_t s);
hipError_t launch_q8_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s);
hipError_t launch_q4_quantize(const float *x, size_t n_blocks, uint8_t *out, hipStream_t s);

}  // namespace q4k
