/*
 * q4k_bench.h -- measurement helpers exported by libq4k.so for the
 * benchmark harness (not part of the compute path).  Same conventions as
 * q4k.h: device pointers owned by the caller, asynchronous on `stream`,
 * return 0 on success, -1 bad size, -2 NULL pointer, -3 misaligned,
 * -4 launch error.
 */
#ifndef Q4K_BENCH_H
#define Q4K_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One empty kernel of one wave: the launch/dispatch floor. */
int q4k_bench_empty(void *stream);

/* One wave that waits about ns nanoseconds (at most 0.1 s) on the GPU's
 * real-time counter, then ends.  Enqueued just before a timed region, it
 * keeps the GPU busy while the host submits the timed work, so the region
 * measures the device's steady rate rather than the host's submission
 * latency. */
int q4k_bench_delay(int64_t ns, void *stream);

/* Streaming read of nbytes (a multiple of 16, src 16-byte aligned) with
 * non-temporal 16-byte loads, grid-stride over at most sink_words
 * workgroups; each workgroup writes one uint32 to sink so the reads stay
 * live.  The achievable read bandwidth for comparison with the GEMVs. */
int q4k_bench_stream_read(const void *src, int64_t nbytes, uint32_t *sink,
                          int64_t sink_words, void *stream);

/* Plain copy of nbytes (multiple of 16, both pointers 16-byte aligned): a
 * kernel of known traffic (nbytes read + nbytes written) used to scale
 * hardware byte counters. */
int q4k_bench_copy(const void *src, void *dst, int64_t nbytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_BENCH_H */
