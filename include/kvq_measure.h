/*
 * kvq_measure.h -- measurement support exported by libkvq.  These calls are not steps of the
 * method; they give the benchmark a measured HBM ceiling (a read-only stream with the same
 * 128-bit loads the decode kernel uses) and a copy kernel of known size against which the
 * hardware byte counters are calibrated.
 *
 * Same conventions as kvq.h: device pointers owned by the caller, asynchronous on `stream`.
 */
#ifndef KVQ_MEASURE_H_
#define KVQ_MEASURE_H_

#include <stddef.h>
#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) from `buf` once with 128-bit loads; each workgroup writes
 * one reduction value to sink[blockIdx] so nothing is optimised away.  `sink` must hold
 * kvq_measure_read_sink_floats() floats.  KVQ_EINVAL / KVQ_EALIGN on bad arguments. */
kvq_status kvq_measure_read(const void *buf, size_t bytes, float *sink, void *stream);
int32_t kvq_measure_read_sink_floats(void);

/* Copy `bytes` (a multiple of 16) from `src` to `dst` with 128-bit loads and stores. */
kvq_status kvq_measure_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_MEASURE_H_ */
