/* Timeline records of the trace build of the library (libmono_decode_trace.so).
 *
 * The trace build is the product library compiled with MONO_TRACE: the same
 * kernels, entry points and results, plus phase stamps that thread 0 of each
 * workgroup writes with the 100 MHz device clock.  Only that library exports
 * these two calls; libmono_decode.so has neither the calls nor the stamps.
 *
 * Records (64-bit words, 32 per record):
 *   items[t * 32 + s]   the work item that took ticket t (t < 8192): stamp 0 =
 *                       start, 1 = end, 2..30 = phases of its kind; word 31 =
 *                       (kind << 24) | item index (kind 1 scan or chunk-local
 *                       chunk, 2 filter slice, 3 attention split, 4 selection,
 *                       255 clear);
 *   groups[w * 32 + s]  workgroup w (w < 4096): stamp 0 = kernel entry, 1 =
 *                       leaving the item loop.
 * Return codes are the MONO_* codes of mono_decode.h.  A stamp that was not
 * reached reads 0.  Records persist across launches until cleared, so clear
 * before the launch to be read.
 */
#ifndef MONO_TRACE_H
#define MONO_TRACE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Zeroes every record (synchronises the device).  Returns MONO_OK or
 * MONO_EHIP. */
int mono_trace_clear(void);

/* Copies the first n_items words of the item records to host `items` and the
 * first n_groups words of the workgroup records to host `groups` (either
 * count may be 0) after a device synchronisation.  n_items <= 8192 * 32,
 * n_groups <= 4096 * 32, else MONO_EINVAL; MONO_EHIP on a HIP failure. */
int mono_trace_read(uint64_t* items, size_t n_items, uint64_t* groups, size_t n_groups);

#ifdef __cplusplus
}
#endif

#endif /* MONO_TRACE_H */
