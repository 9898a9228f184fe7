/*
 * q4_probe.h — measurement-only companion library (libq4probe.so) of libq4.
 *
 * It holds no part of the block-quantized method. Its one kernel reads a
 * buffer with plain 16-byte loads, every load of a thread issued up front,
 * and nothing else, so its time over the same bytes, in the same harness and
 * cache state as a GEMV, is the practical ceiling against which the GEMV's
 * HBM fraction can be read (the streaming-
 * read ceiling of the measurement plan; compare "fuel-vulkan-kernels —
 * quantized (GGML) kernel contracts", section qmatvec_q4_0, which bounds the
 * GEMV by streaming the weight blocks once).
 */
#ifndef Q4_PROBE_H
#define Q4_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * q4probe_stream_read — read bytes [src, src + n_bytes) once, with 16-byte
 * loads, on `stream` (a hipStream_t; NULL is the default stream).
 *   src       device pointer, 16-byte aligned; n_bytes a multiple of 16.
 *   sink      device pointer to 16 bytes, written only if the XOR of all the
 *             data equals a fixed constant (so the loads cannot be removed).
 * Returns 0 on success, 1 for a NULL pointer, 2 for more than 4 GiB, 3 for
 * n_bytes % 16 != 0, 4 for a misaligned pointer, 6 if the launch is refused.
 * n_bytes == 0 launches nothing.
 */
int q4probe_stream_read(const void *src, size_t n_bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
