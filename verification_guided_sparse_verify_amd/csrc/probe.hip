// Streaming-read ceiling probe (libvegas_probe.so): measurement only, shares
// nothing with the Vegas kernels.  See include/vegas_probe.h.
#include <hip/hip_runtime.h>

#include "vegas_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;     // 1 KB wave-wide copies per wave per round
constexpr size_t kRoundBytes = (size_t)16 * kThreads * kInFlight;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Each wave streams its part of the workgroup's slice into its own 8 KB of
// LDS with 16-byte direct-to-LDS copies (non-temporal policy), eight in
// flight, then waits for all of them before the next round.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const unsigned char* __restrict__ src,
                                                               size_t per_wg, uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint4 buf[kThreads * kInFlight];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const unsigned char* base = src + (size_t)blockIdx.x * per_wg + (size_t)wave * 1024 * kInFlight + 16 * lane;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)(buf + wave * 64 * kInFlight);
    for (size_t off = 0; off < per_wg; off += kRoundBytes) {
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const unsigned char* p = base + off + (size_t)u * 1024;
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(p), "{m0}"(lds0 + 1024u * u)
                         : "memory");
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // Fold the last round; one lane per workgroup reports only a zero fold
    // (never, for data of any interest).
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
        const uint4 v = buf[u * kThreads + threadIdx.x];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0u && threadIdx.x == 0) sink[blockIdx.x] = 1u;
}

}  // namespace

extern "C" int vegas_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                       void* stream) {
    if (!src || !sink || workgroups < 1 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return -1;
    const size_t unit = kRoundBytes * (size_t)workgroups;
    if (bytes == 0 || bytes % unit != 0) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(src), bytes / (size_t)workgroups, sink);
    return (int)hipGetLastError();
}
