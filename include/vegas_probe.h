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

#ifdef __cplusplus
}
#endif

#endif
