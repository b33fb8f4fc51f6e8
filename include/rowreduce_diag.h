/*
 * rowreduce_diag.h -- the diagnostics build of the library,
 * librowreduce_diag.so: every entry point of rowreduce.h (the same kernel
 * object, linked unchanged, so the same kernels and bits) plus three entry
 * points for tests and measurement that the product library
 * librowreduce.so does not carry:
 *   rr_set_variant_override     force a kernel variant (process-wide state)
 *   rr_selftest_wave_allreduce  run the wave64 all-reduce on given lanes
 *   rr_stream_copy              a plain streaming copy, the practical
 *                               bandwidth bar beside each operation
 *   rr_set_split_wait_ticks     shorten the one-kernel split's wait
 *   rr_split_fallbacks          how often that wait expired
 * Conventions (device pointers, streams, errors) as in rowreduce.h.
 */
#ifndef ROWREDUCE_DIAG_H
#define ROWREDUCE_DIAG_H

#include "rowreduce.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Forced kernel variant, process-wide, for tests and measurement
 * (RR_VARIANT_AUTO restores the automatic choice).  Every call of this
 * library, rr_query_plan included, then plans with that variant; a forced
 * variant that cannot run a shape makes that call return
 * RR_ERR_UNSUPPORTED.  It is state of this diagnostics build only: calls in
 * flight on other threads see the change at an unspecified point. */
rr_status rr_set_variant_override(rr_variant variant);

/*
 * Self-test of the wave64 all-reduce (device work; used by the test suite).
 * kind 0: in and out hold count groups of 64 floats; every lane of a group
 * receives the group's sum.  kind 1: the same with the maximum.  kind 2: in
 * and out hold count groups of 128 floats, 64 m values then 64 d values;
 * every lane receives the merge of the group's 64 (m, d) pairs.  One
 * wavefront per group; 1 <= count <= (2^32 - 1) / 64.
 */
rr_status rr_selftest_wave_allreduce(const float* in, float* out, int64_t count, int kind,
                                     void* stream);

/*
 * Streaming copy, a measurement reference rather than an operation of the
 * method: dst[0, bytes) <- src[0, bytes) with 16-byte non-temporal loads and
 * stores, one vector per lane, no dependency between elements.  An operation
 * that reads B/2 bytes and writes B/2 bytes moves the same HBM traffic as a
 * copy of B/2 bytes, so the copy's speed at that size is the practical
 * streaming bar to set the operation's speed beside (the fixed start-up and
 * drain of a launch are a visible share at a few hundred megabytes).
 *   dst, src  device pointers, 16-byte aligned, not overlapping
 *   bytes     >= 0, a multiple of 16 (0: no launch)
 * Returns RR_ERR_INVALID_ARG for a bad size, null or misaligned pointers, or
 * overlap; asynchronous on `stream` like every other call.
 */
rr_status rr_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * The split softmax in one kernel (RR_VARIANT_SPLIT in rowreduce.h): each
 * workgroup waits a bounded time for the other chunks' (m, d) summaries of
 * its row and summarises a chunk again from x itself when one has not
 * arrived, so the result has the same bits either way.  Each such chunk adds
 * one to a counter per device.
 *   rr_set_split_wait_ticks  the wait, in ticks of the 100 MHz real-time
 *                            clock, for every later call of this library
 *                            (process-wide; default 4000 = 40 us; at most
 *                            10^8); 0 gives up at once whenever a summary is
 *                            not there yet, which exercises the fallback.
 *   rr_split_fallbacks       *count <- the current device's counter (after
 *                            a device-wide synchronisation); reset != 0
 *                            then clears it.  Synchronous.
 */
rr_status rr_set_split_wait_ticks(uint64_t ticks);
rr_status rr_split_fallbacks(uint32_t* count, int reset);

#ifdef __cplusplus
}
#endif

#endif /* ROWREDUCE_DIAG_H */
