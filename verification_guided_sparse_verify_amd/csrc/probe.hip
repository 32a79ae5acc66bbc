// Streaming-read ceiling probe (libvegas_probe.so): measurement only, shares
// nothing with the Vegas kernels.  See include/vegas_probe.h.
#include <hip/hip_runtime.h>

#include "vegas_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;     // 16-byte loads per thread per round

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint4* __restrict__ src, size_t per_wg16,
                                                               uint32_t* __restrict__ sink) {
    const uint4* base = src + (size_t)blockIdx.x * per_wg16;
    uint32_t acc = 0;
    for (size_t i = threadIdx.x; i < per_wg16; i += (size_t)kThreads * kInFlight) {
        uint4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            v[u] = j < per_wg16 ? base[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one lane per workgroup reports only a zero fold (never, for data of any
    // interest), which keeps the loads live without a store per thread
    if (acc == 0u && threadIdx.x == 0) sink[blockIdx.x] = 1u;
}

}  // namespace

extern "C" int vegas_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                       void* stream) {
    if (!src || !sink || workgroups < 1 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return -1;
    const size_t unit = (size_t)16 * workgroups * kThreads;
    if (bytes == 0 || bytes % unit != 0) return -1;
    const size_t per_wg16 = bytes / 16 / (size_t)workgroups;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(src), per_wg16, sink);
    return (int)hipGetLastError();
}
