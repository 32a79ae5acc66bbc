// Measurement probes (libvegas_probe.so): streaming and gathered read
// ceilings and the dependent-launch floor; they share nothing with the Vegas
// kernels.  See include/vegas_probe.h.
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

// Gathered reads: the K and V slices (SLICE bytes of head h) of listed token
// rows, the access pattern of the drafting pass, with no arithmetic.  A
// workgroup takes head w % heads and the w / heads-th range of `per_wg` list
// entries (at most kGatherMaxRange), stages the range's row numbers in LDS,
// and its waves stream 16-row blocks in turn through private rings of DEPTH
// blocks (16-byte direct-to-LDS copies, non-temporal policy): a block is
// awaited while the next DEPTH-1 are in flight, as the drafting pass's ring
// does.  Row numbers are clamped into [0, total_rows).
constexpr int kGatherRows = 16;
constexpr int kGatherMaxRange = 4096;
// HPW heads per workgroup: wave w reads head HPW * (workgroup % groups) + w % HPW
// and takes the 16-row blocks w / HPW, w / HPW + 4 / HPW, ... of the
// workgroup's range; each wave waits for its oldest block, then issues the
// next, keeping DEPTH - 1 blocks in flight, and issues nothing past its last.
template <int SLICE, int DEPTH, int HPW>
__global__ void __launch_bounds__(kThreads) gather_read_kernel(const unsigned char* __restrict__ k,
                                                               const unsigned char* __restrict__ v,
                                                               const int32_t* __restrict__ rows, int32_t n_rows,
                                                               int32_t total_rows, int32_t row_bytes, int32_t heads,
                                                               int32_t per_wg, uint32_t* __restrict__ sink) {
    constexpr int CPR = SLICE / 16;                // 16-byte chunks per row slice
    constexpr int RPC = 64 / CPR;                  // rows per wave-wide copy
    constexpr int COPIES = kGatherRows / RPC;      // copies per tensor per block
    constexpr int BLK = kGatherRows * SLICE;       // bytes per tensor per block
    constexpr int OPS = 2 * COPIES;                // copies per block
    constexpr int NPG = 4 / HPW;                   // waves per head
    static_assert(DEPTH >= 2 && DEPTH <= 4, "one to three blocks in flight");
    __shared__ __attribute__((aligned(16))) unsigned char ring[kThreads / 64][DEPTH][2 * BLK];
    __shared__ int idx_s[kGatherMaxRange];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int groups = heads / HPW;
    const int head = HPW * (blockIdx.x % groups) + wave % HPW;
    const int pg = wave / HPW;
    const int first = (blockIdx.x / groups) * per_wg;
    const int count = max(min(first + per_wg, n_rows) - first, 0);
    for (int i = threadIdx.x; i < count; i += kThreads) idx_s[i] = min(max(rows[first + i], 0), total_rows - 1);
    __syncthreads();
    const int nblk = (count + kGatherRows - 1) / kGatherRows;
    const int mine = pg < nblk ? (nblk - pg + NPG - 1) / NPG : 0;   // this wave's blocks: pg, pg + NPG, ...
    auto issue = [&](int j, int stage) {
        const int blk = pg + NPG * j;
#pragma unroll
        for (int c = 0; c < COPIES; ++c) {
            const int e = min(blk * kGatherRows + c * RPC + lane / CPR, count - 1);
            const size_t off = (size_t)idx_s[e] * (uint32_t)row_bytes + (size_t)head * SLICE + (lane % CPR) * 16;
            const uint32_t lk = (uint32_t)(uintptr_t)(lds_ptr_t)(&ring[wave][stage][c * 1024]);
            const uint32_t lv = (uint32_t)(uintptr_t)(lds_ptr_t)(&ring[wave][stage][BLK + c * 1024]);
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(k + off), "{m0}"(lk) : "memory");
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(v + off), "{m0}"(lv) : "memory");
        }
    };
    uint32_t acc = 0;
    if (mine > 0) {
#pragma unroll
        for (int j = 0; j < DEPTH - 1; ++j)
            if (j < mine) issue(j, j);
        for (int j = 0; j < mine; ++j) {
            // block j has landed: the copies of the blocks after it that were issued may still fly
            const int after = min(DEPTH - 2, mine - 1 - j);
            if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * OPS) : "memory");
            else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(OPS) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (j + DEPTH - 1 < mine) issue(j + DEPTH - 1, (j + DEPTH - 1) % DEPTH);
            acc ^= reinterpret_cast<const uint32_t*>(&ring[wave][j % DEPTH][0])[lane];
        }
    }
    if (acc == 0u && lane == 0 && mine > 0 && blockIdx.x == 0x7fffffff) sink[0] = 1u;   // keeps the reads live
}

__global__ void __launch_bounds__(kThreads) launch_chain_kernel(uint32_t* __restrict__ sink) {
    extern __shared__ uint32_t chain_lds[];
    if (blockIdx.x == 0 && threadIdx.x == 0) sink[0] = sink[0] + 1u;
    (void)chain_lds;
}

// Spins one wave for `ticks` of the 100 MHz constant clock (bounded: the clock
// only moves forward), so that launches queued behind it are timed on the GPU
// alone.
__global__ void __launch_bounds__(64) delay_kernel(unsigned long long ticks, uint32_t* __restrict__ sink) {
    const unsigned long long t0 = wall_clock64();
    unsigned long long t = t0;
    while (t - t0 < ticks) t = wall_clock64();
    if (threadIdx.x == 0) sink[0] = sink[0] + (uint32_t)(t - t0 > ticks);
}

}  // namespace

extern "C" int vegas_probe_delay(int64_t ticks, uint32_t* sink, void* stream) {
    if (!sink || ticks < 0 || ticks > 100000000) return -1;
    hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       (unsigned long long)ticks, sink);
    return (int)hipGetLastError();
}

extern "C" int vegas_probe_launch_chain(int32_t launches, int32_t workgroups, int32_t lds_bytes, uint32_t* sink,
                                        void* stream) {
    if (!sink || launches < 1 || launches > 100000 || workgroups < 1 || workgroups > 4096 || lds_bytes < 0 ||
        lds_bytes > 65536)
        return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    for (int i = 0; i < launches; ++i)
        hipLaunchKernelGGL(launch_chain_kernel, dim3(workgroups), dim3(kThreads), (size_t)lds_bytes, st, sink);
    return (int)hipGetLastError();
}

extern "C" int vegas_probe_gather_read(const void* k, const void* v, const int32_t* rows, int32_t n_rows,
                                       int32_t total_rows, int32_t row_bytes, int32_t slice_bytes, int32_t heads,
                                       int32_t heads_per_workgroup, int32_t workgroups, int32_t blocks_in_flight,
                                       uint32_t* sink, void* stream) {
    if (!k || !v || !rows || !sink || n_rows < 1 || total_rows < 1 || heads < 1 || blocks_in_flight < 1 ||
        blocks_in_flight > 3 || (heads_per_workgroup != 1 && heads_per_workgroup != 2) ||
        heads % heads_per_workgroup != 0)
        return -1;
    const int groups = heads / heads_per_workgroup;
    if (workgroups < groups || workgroups % groups != 0) return -1;
    if ((slice_bytes != 128 && slice_bytes != 256) || row_bytes < heads * slice_bytes || row_bytes % 16 != 0)
        return -1;
    if (((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u) != 0) return -1;
    const int per_group = workgroups / groups;
    const int per_wg = (n_rows + per_group - 1) / per_group;
    if (per_wg > kGatherMaxRange) return -1;
    const dim3 grid(workgroups), block(kThreads);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const unsigned char* kb = static_cast<const unsigned char*>(k);
    const unsigned char* vb = static_cast<const unsigned char*>(v);
#define VEGAS_PROBE_GATHER(S, D, H)                                                                             \
    hipLaunchKernelGGL((gather_read_kernel<S, D, H>), grid, block, 0, st, kb, vb, rows, n_rows, total_rows,     \
                       row_bytes, heads, per_wg, sink)
#define VEGAS_PROBE_GATHER_D(S, H)                 \
    do {                                           \
        if (depth == 2) VEGAS_PROBE_GATHER(S, 2, H); \
        else if (depth == 3) VEGAS_PROBE_GATHER(S, 3, H); \
        else VEGAS_PROBE_GATHER(S, 4, H);          \
    } while (0)
    const int depth = blocks_in_flight + 1;       // ring stages: blocks in flight plus the one awaited
    if (slice_bytes == 256) {
        if (heads_per_workgroup == 1) VEGAS_PROBE_GATHER_D(256, 1);
        else VEGAS_PROBE_GATHER_D(256, 2);
    } else {
        if (heads_per_workgroup == 1) VEGAS_PROBE_GATHER_D(128, 1);
        else VEGAS_PROBE_GATHER_D(128, 2);
    }
#undef VEGAS_PROBE_GATHER_D
#undef VEGAS_PROBE_GATHER
    return (int)hipGetLastError();
}

extern "C" int vegas_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                                       void* stream) {
    if (!src || !sink || workgroups < 1 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0) return -1;
    const size_t unit = kRoundBytes * (size_t)workgroups;
    if (bytes == 0 || bytes % unit != 0) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const unsigned char*>(src), bytes / (size_t)workgroups, sink);
    return (int)hipGetLastError();
}
