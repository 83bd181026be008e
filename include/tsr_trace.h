/*
 * tsr_trace.h - phase stamps of the tracing build of the sampler library
 * (libtsr_trace.so, built with TSR_TRACE=1 by build.py --trace). The ordinary
 * libtsr.so neither stamps nor exports these calls.
 *
 * Each wavefront of the first 4096 workgroups of a traced launch writes the
 * device's 100 MHz real-time counter at fixed points of the sampler kernels
 * (slots 0-10: entry, loads issued, pass A done, row statistics, first
 * compaction, top-k bound, second compaction, fast resolve, register search,
 * walk, outputs written; a slot a row does not reach keeps its old value) to
 * a buffer the handle owns: entry ((block * waves_per_block + wave) * 16 +
 * slot) of 4096 * 16 * 16 unsigned 64-bit words. Only sample_rows and its
 * variants stamp.
 */
#ifndef TSR_TRACE_H_
#define TSR_TRACE_H_

#include <stdint.h>

#include "tsr.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of 64-bit words of the handle's stamp buffer. */
#define TSR_TRACE_WORDS (4096 * 16 * 16)

/* Wait for the device, then copy the first n (<= TSR_TRACE_WORDS) words of
 * the handle's stamp buffer to host memory `out`. TSR_EINVAL on a null
 * handle or out, or n out of range. */
int sampler_trace_read(tsr_handle h, uint64_t* out, int64_t n);

/* Wait for the device and set every word of the stamp buffer to 0. */
int sampler_trace_clear(tsr_handle h);

#ifdef __cplusplus
}
#endif

#endif /* TSR_TRACE_H_ */
