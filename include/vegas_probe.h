/*
 * vegas_probe.h -- measurement helper of libvegas_probe.so (built next to
 * libvegas.so).  Not part of the Vegas path: it gives the benchmark a measured
 * "practical peak" of HBM reads on the device at hand, next to the published
 * 8 TB/s, for the roofline fraction of the bandwidth-bound kernels.
 */
#ifndef VEGAS_PROBE_H
#define VEGAS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes of device memory from `src` (16-byte
 * aligned, bytes a multiple of 32768 * workgroups) by `workgroups`
 * workgroups of 256 threads: workgroup w reads the w-th equal contiguous
 * slice in rounds of 32 KB, each of its four waves copying 8 KB into its own
 * LDS with eight 16-byte-per-lane direct-to-LDS loads in flight under the
 * non-temporal cache policy (the load path of the attention kernels).  The
 * last round is folded into sink[w] (device uint32 [workgroups]; written only
 * for an all-zero fold).  Asynchronous on `stream`.  Returns 0, or -1 for
 * invalid arguments (nothing launched), or the HIP error code of the launch.
 */
int vegas_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/*
 * Gathered read of the drafting pass's bytes with no arithmetic: for every
 * entry e of rows (device int32 [n_rows], token row numbers, clamped into
 * [0, total_rows)), the slice_bytes-byte slice of each of `heads` heads of
 * row rows[e] of k and of v (row r, head h at byte r * row_bytes +
 * h * slice_bytes).  Workgroups take heads_per_workgroup (1 or 2, dividing
 * heads) heads each: workgroup w (of `workgroups`, a multiple of
 * heads / heads_per_workgroup) reads an equal range of at most 4096 entries,
 * whose row numbers it stages in LDS first; with two heads, waves 2i and
 * 2i+1 read the two heads' slices of the same rows (the drafting kernel's
 * head pairs).  Each wave takes its head's 16-row blocks in turn through a
 * private ring: it waits for its oldest block, then issues the next, keeping
 * blocks_in_flight (1..3) blocks in flight, with 16-byte direct-to-LDS
 * copies under the non-temporal cache policy and nothing past its last
 * block.  slice_bytes is 128 or 256; k and v 16-byte aligned.  sink: device
 * uint32 [1], never written in practice (it keeps the reads live).
 * Asynchronous on `stream`.  Returns 0, -1 for invalid arguments (nothing
 * launched), or the HIP error code of the launch.
 */
int vegas_probe_gather_read(const void* k, const void* v, const int32_t* rows, int32_t n_rows, int32_t total_rows,
                            int32_t row_bytes, int32_t slice_bytes, int32_t heads, int32_t heads_per_workgroup,
                            int32_t workgroups, int32_t blocks_in_flight, uint32_t* sink, void* stream);

/*
 * Dependent-launch floor: `launches` (1..100000) launches back to back on
 * `stream` of a kernel with `workgroups` (1..4096) workgroups of 256 threads
 * and lds_bytes (0..65536) of LDS each, that does no work except that its
 * first thread increments sink[0] (device uint32 [1]), so each launch reads
 * what the one before wrote.  The time of a long chain divided by `launches`
 * is the cost of one kernel boundary in a chain of dependent launches on one
 * stream (dispatch, workgroup start-up and drain, end-of-kernel cache
 * write-back): the floor under each of a pass's small dependent kernels.
 * Asynchronous.  Returns 0, -1 for invalid arguments (nothing launched), or
 * the HIP error code of the last launch.
 */
int vegas_probe_launch_chain(int32_t launches, int32_t workgroups, int32_t lds_bytes, uint32_t* sink, void* stream);

/*
 * One wave on `stream` that spins for `ticks` (0..1e8, i.e. up to 1 s) of the
 * 100 MHz constant clock and then adds 0 or 1 to sink[0] (device uint32 [1]).
 * Launched before a timed chain, it holds the GPU while the host queues the
 * chain, so the chain's time is the GPU's own and not the host's launch rate.
 * Asynchronous.  Returns 0, -1 for invalid arguments (nothing launched), or the
 * HIP error code of the launch.
 */
int vegas_probe_delay(int64_t ticks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif
