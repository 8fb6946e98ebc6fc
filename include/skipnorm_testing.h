/*
 * skipnorm_testing.h -- route-selection and measurement hooks of libskipnorm.
 *
 * Not part of the operator interface (skipnorm.h): these let tests run every
 * kernel family on the same shapes, force the exchange's fallback path, and
 * give benchmarks a copy kernel of known traffic.  They change process-wide
 * settings; production callers need none of them.
 */
#ifndef SKIPNORM_TESTING_H
#define SKIPNORM_TESTING_H

#include "skipnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Route selection for every later call in the process:
 *   0 = automatic (the default);
 *   1 = element-by-element accesses (vectors off);
 *   2 = vectorized where the preconditions hold (same as automatic, except
 *       that gated_rms_norm keeps one power-of-two lane group per row for
 *       every row length, where automatic packs rows that are not a power
 *       of two of vectors back to back);
 *   3 = skip_rms_norm / skip_layer_norm / gated_rms_norm: one workgroup per
 *       row, two passes, element by element;
 *       skip_group_norm: the three-launch split route with scalar accesses;
 *   4 = skip_group_norm: the three-launch split route (vectorized where the
 *       preconditions hold) even where a single-launch route would apply;
 *       others: automatic.
 *   5 = gated_rms_norm, skip_rms_norm, skip_layer_norm: the flat route
 *       (rows read as one stream of aligned 16-byte vectors) wherever it
 *       applies -- rows of at most 1016 (float16) or 1020 (float32)
 *       elements (skip_layer_norm: at least 3), the data tensors (X, gate,
 *       Y; input, skip, output, S) at one offset from a 16-byte boundary --
 *       where automatic takes it only for the row lengths it measured
 *       faster on; skip_group_norm: automatic.
 * Returns the previous value; an unknown value leaves the setting unchanged
 * and returns the current one. */
int skipnorm_force_route(int route);

/* SkipGroupNorm's single-launch routes spread each (n, group) over several
 * workgroups (NCHW: up to 8; NHWC: up to 64 pixel slices of an image) that
 * exchange partial moments; a workgroup waits at most this long for
 * another's moments and otherwise recomputes them itself with the same
 * arithmetic (results are identical either way).  Sets the wait for
 * later calls in the process (negative: the default, 100 us) and returns the
 * previous value.  0 forces every recomputation path. */
int skipnorm_set_exchange_timeout_us(int microseconds);

/* Name of the route the calling thread's last successful op call took
 * (e.g. "ssln.wave2.vec16", "ssln.segment.vec8", "gated.tile.vec8",
 * "sgn.cluster.nhwc.vec16", "sgn.split.nchw.scalar"). */
const char* skipnorm_last_route(void);

/* Measurement helper: copies `bytes` bytes from src to dst with one kernel
 * of 16-byte loads and stores (both 16-byte aligned, bytes a multiple of
 * 16).  Serves as the copy-bandwidth reference and as the calibration
 * kernel of known traffic for hardware counters. */
sn_status skipnorm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SKIPNORM_TESTING_H */
