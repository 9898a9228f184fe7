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

/*
 * q4probe_stream_read_cfg — the same read with a chosen launch shape, for
 * sweeping it: `threads` per workgroup (64, 128, 256, 512 or 1024), `loads`
 * 16-byte loads per thread, all issued before any is used (1, 2, 4, 8 or 16;
 * the grid is ceil(n_bytes / (16 threads loads)) workgroups), and `flags`:
 * bit 0 non-temporal loads, bit 1 blocked (each workgroup reads one
 * contiguous run of 16 threads loads bytes; otherwise a thread's loads are a
 * grid's width apart). Returns as q4probe_stream_read, and 5 for a shape
 * outside those sets. q4probe_stream_read is this with 512 threads, one load
 * and non-temporal loads, the sweep's fastest shape.
 */
int q4probe_stream_read_cfg(const void *src, size_t n_bytes, void *sink, int threads, int loads,
                            int flags, void *stream);

/*
 * q4probe_stream_rw — read groups * read_words and write groups * write_words
 * 16-byte words in that proportion, evenly interleaved (one wavefront per
 * group of read_words words in and write_words words out, max of the two 64),
 * with non-temporal loads and stores: the read-and-write ceiling for a kernel
 * that turns one block stream into another of a different size (Q8_0
 * quantize: 64 words read per 17 written; Q4_0 dequant: 9 per 64). Each
 * wavefront takes `loads` groups (1, 2, 4 or 8) a grid's width apart, all
 * loads issued before any store; `flags` bit 0 makes the loads and bit 1 the
 * stores non-temporal. The fastest of these shapes is the ceiling.
 *   src       groups * read_words * 16 bytes, read once.
 *   dst       groups * write_words * 16 bytes, every byte written once with a
 *             copy of a word of src (contents not meaningful).
 *   sink      as q4probe_stream_read.
 * Returns 0 on success (groups == 0 launches nothing), 1 for a NULL pointer,
 * 2 for more than 4 GiB on either side, 4 for a misaligned pointer, 5 for
 * word counts outside [1, 64] or with neither equal to 64, another `loads`
 * or other flag bits, 6 if the launch is refused.
 */
int q4probe_stream_rw(const void *src, void *dst, size_t groups, int read_words, int write_words,
                      int loads, int flags, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif
