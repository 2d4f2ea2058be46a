/*
 * attn_probe.h -- HBM bandwidth probes for the roofline of the HBM-bound
 * kernels (decode, the sliding-window prefill).  Measurement only: no step of
 * the attention path calls them.  They stream a buffer with 16-byte
 * non-temporal loads (and stores), every workgroup taking one contiguous chunk
 * (as a decode split takes its keys) in steps of whole KB per wave, a grid of
 * up to 16 workgroups per CU: the rate they reach is what this GPU sustains
 * for streaming access.
 *
 * Pointers are device pointers, 16-byte aligned; `bytes` a multiple of 16.
 * Calls are enqueued on `stream` (NULL = the default stream) and return an
 * attn_status code of attn.h: ATTN_ERR_NULL, ATTN_ERR_ALIGN or ATTN_ERR_SHAPE
 * for bad arguments (checked before any HIP call), ATTN_ERR_HIP if the launch
 * fails.  bytes = 0 does nothing.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words attn_probe_read writes to `sink` for a buffer of `bytes` bytes (one
 * 32-bit fold of the data per wave, so that no load is optimised away). */
size_t attn_probe_sink_words(size_t bytes);

/* Read `bytes` bytes of src once; sink receives attn_probe_sink_words(bytes)
 * words (caller-owned device memory). */
int attn_probe_read(const void* src, size_t bytes, unsigned int* sink, void* stream);

/* Copy `bytes` bytes from src to dst (non-overlapping): bytes read + written
 * = 2 * bytes. */
int attn_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
