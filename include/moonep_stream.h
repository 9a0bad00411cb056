/*
 * moonep_stream.h -- streaming kernels that measure the practical HBM ceilings
 * of one MI355X (gfx950): what a plain sequential read, write or copy of a
 * device buffer sustains. They are not part of the method; the benchmark times
 * them on the same buffers as the data moves (dispatch, combine) so that every
 * move can be stated as a fraction of both the 8 TB/s peak and these ceilings.
 * Built as its own library, libmoonep_stream.so.
 *
 * Conventions: device pointers owned by the caller, 16-byte aligned, `bytes` a
 * positive multiple of 16; the call only enqueues one kernel on `stream` (a
 * hipStream_t passed as void*) and never synchronises or allocates.
 * chunk_bytes picks the launch shape: 0 = one resident grid that walks the whole
 * buffer with a grid-stride loop; a positive multiple of 4096 = one 256-thread
 * workgroup per contiguous chunk of that many bytes.
 * Returns 0, -1 (bytes not a positive multiple of 16, or a bad chunk_bytes), -2
 * (NULL or misaligned pointer) or -3 (the launch failed).
 */
#ifndef MOONEP_STREAM_H
#define MOONEP_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of src once with 16-byte non-temporal loads. The loaded
   values are folded into a per-lane word that is stored to sink (16 bytes) only
   if it equals a fixed constant, so the loads cannot be dropped while the
   kernel writes (almost) nothing. */
int moonep_stream_read(const void *src, int64_t bytes, int64_t chunk_bytes, void *sink,
                       void *stream);

/* Writes `pattern` to every 32-bit word of dst with 16-byte stores. */
int moonep_stream_write(void *dst, int64_t bytes, int64_t chunk_bytes, uint32_t pattern,
                        void *stream);

/* dst = src byte for byte (16-byte non-temporal loads, plain stores); the two
   ranges must not overlap. */
int moonep_stream_copy(void *dst, const void *src, int64_t bytes, int64_t chunk_bytes,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_STREAM_H */
