/*
 * dsa_calib.h - measurement helpers shipped beside the selector library.
 *
 * None of these is part of candidate-block selection.  The benchmark uses
 * them to put its numbers in context on the same GPU:
 *   - a plain device copy of known size, whose hardware read/write byte
 *     counters give the scale factor for the selector's counters;
 *   - a read-only stream, the bandwidth a pure HBM read reaches on this machine;
 *   - a write-only stream (fill), the same for pure writes;
 *   - an empty kernel, the launch floor of back-to-back calls.
 * Same conventions as dsa.h: caller-owned buffers, work enqueued on `stream`,
 * no synchronisation, 0 on success, otherwise a dsa_status_t code
 * (1 = invalid argument, 4 = HIP error).
 */
#ifndef DSA_CALIB_H
#define DSA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0, bytes) = src[0, bytes); both 16-byte aligned, bytes % 16 == 0. */
int dsa_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Reads src[0, bytes) once (16-byte aligned, bytes % 16 == 0).  The xor of
 * what each workgroup read decides whether it stores one uint32 into
 * sink[0, dsa_calib_read_sink_words()), so the reads cannot be elided; the
 * sink's contents are meaningless. */
int dsa_calib_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
size_t dsa_calib_read_sink_words(void);

/* dst[0, bytes) = `word` repeated (16-byte aligned, bytes % 16 == 0); with
 * word = 0xFF800000 that is fp32 -inf. */
int dsa_calib_fill(void* dst, size_t bytes, uint32_t word, hipStream_t stream);

/* One launch of a kernel that does nothing (one workgroup). */
int dsa_calib_empty(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_CALIB_H */
