/*
 * spec_measure.h -- measurement hooks of libspecverify.so.
 *
 * Not part of the verification method: these calls exist so that a benchmark
 * can time each library kernel with HIP events on the stream it runs on, and
 * can calibrate bandwidth figures against plain streaming kernels.
 */
#ifndef SPEC_MEASURE_H
#define SPEC_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on its launch stream.  Process-wide; not for use while
 * other threads call the library.  Enabling creates events (host allocation). */
spec_status_t spec_timing_enable(int enable);

/* Drop every recorded launch. */
spec_status_t spec_timing_reset(void);

/* Waits for the recorded events, then aggregates them per kernel name.
 * Returns the number of distinct kernel names recorded since the last reset. */
int spec_timing_collect(void);

/* Entry `index` (0 <= index < spec_timing_collect()) of the aggregate:
 * kernel name (static storage), number of launches, summed milliseconds. */
spec_status_t spec_timing_entry(int index, const char** name, long long* launches, double* total_ms);

/* Read-only streaming probe: sums `bytes` (a multiple of 16, 16-byte aligned)
 * of device memory at `src` as 32-bit words into *out (device uint32). */
spec_status_t spec_probe_read(const void* src, size_t bytes, uint32_t* out, spec_stream_t stream);

/* Plain copy of `bytes` (a multiple of 16, 16-byte aligned) from src to dst. */
spec_status_t spec_probe_copy(const void* src, void* dst, size_t bytes, spec_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_MEASURE_H */
