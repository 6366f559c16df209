/*
 * pa_probe.h -- C-ABI of the decode bench's measurement kernels (gfx950).
 *
 * Not part of the decode path: two plain kernels with a known number of HBM
 * bytes, which the bench uses to state the practical read ceiling of the
 * device and to scale hardware byte counters.
 *
 * All pointers are DEVICE memory owned by the caller, 16-byte aligned;
 * `bytes` is a positive multiple of 16.  Calls are asynchronous on `stream`
 * (a hipStream_t; NULL = the null stream).  Each returns PA_PROBE_OK (0) or a
 * negative PA_PROBE_ERR_* code, checked on the host before any launch.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_PROBE_OK 0
#define PA_PROBE_ERR_ARG (-1)    /* NULL or misaligned pointer, bad size */
#define PA_PROBE_ERR_LAUNCH (-5) /* no usable device or launch error */

/*
 * Reads buf[0 .. bytes) once with 16-byte loads (a coalesced stream).  `sink`
 * (at least 1 KiB) is written only in the rare case the XOR of all words read
 * equals a fixed value; it exists so that the loads cannot be optimised away.
 */
int pa_probe_read(const void *buf, int64_t bytes, void *sink, void *stream);

/* Copies src[0 .. bytes) to dst (non-overlapping): reads and writes `bytes`. */
int pa_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
