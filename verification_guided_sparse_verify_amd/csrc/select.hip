// Exact top-k KV selection for gfx950.
//
// The selected set (gist.science summary of Vegas, sec. 2A) is the k prefix
// positions with the largest score summed over collected rows and query
// heads.  The verification kernel leaves one fp32 sum per (KV head, position);
// here S[i] = sum over KV heads, then an exact radix select on the
// order-preserving 32-bit image of S:
//
//   pass 1 (many workgroups per sequence): S, its key, a 12-bit histogram of
//           the top digit in LDS, merged into a per-sequence global histogram;
//   pass 2 (one workgroup per sequence):
//     a. from the histogram: the top digit d1 that holds the k-th largest key;
//     b. ordered compaction of every position whose top digit is >= d1 (a
//        superset of T, about k plus one histogram bin) into a scratch list,
//        in ascending position order;
//     c. two 10-bit refinement histograms over that list give the exact k-th
//        largest key theta and how many positions equal to theta to take;
//     d. ordered compaction of the list: key > theta, or key == theta among
//        the first ones in position order -> ascending T.
// Ordered compaction uses wave ballots and lane-prefix popcounts; workgroup
// offsets go through LDS with one barrier per 8192 positions.
#include "internal.h"

namespace vegas {
namespace {

constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / 64;
constexpr int kPer = 8;                       // consecutive items per thread per round
constexpr int kRound = kFinishThreads * kPer;

__device__ __forceinline__ uint32_t order_key(float f) {
    f = f + 0.0f;                             // -0 and +0 share one key
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void sel_zero_kernel(uint32_t* __restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

__global__ void __launch_bounds__(256) sel_keys_kernel(const SelectArgs a) {
    __shared__ uint32_t h[kSelBins];
    const int b = blockIdx.y;
    const int seq0 = a.cu_seqlens_k[b];
    const int L = a.cu_seqlens_k[b + 1] - seq0 - a.W;
    const int start = blockIdx.x * kSelChunk;
    if (start >= L) return;
    const int end = min(start + kSelChunk, L);
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int p = start + threadIdx.x; p < end; p += blockDim.x) {
        const size_t col = (size_t)seq0 + p;
        float s = 0.f;
        for (int g = 0; g < a.hkv; ++g) s += a.scores[(size_t)g * a.total_kv + col];
        const uint32_t key = order_key(s);
        a.keys[col] = key;
        atomicAdd(&h[key >> (32 - kSelDigitBits)], 1u);
    }
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)b * kSelBins;
    for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Exclusive prefix sum over the workgroup's threads in thread order.
__device__ __forceinline__ int wg_exclusive_scan(int x, int* wsum, int* total) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off);
        if (lane >= off) v += y;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < kFinishWaves; ++i) {
        const int t = wsum[i];
        before += (i < w) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + v - x;
}

// Position of every true predicate among all true predicates of the round,
// items ordered by (thread, item).  Returns the round's total.
__device__ __forceinline__ int round_offsets(const bool (&pred)[kPer], int (&off)[kPer], int* wsum) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int lower_lanes = 0, wave_total = 0, mine = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const uint64_t bal = __ballot(pred[e]);
        lower_lanes += __popcll(bal & below);
        wave_total += __popcll(bal);
    }
    if (lane == 0) wsum[w] = wave_total;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < kFinishWaves; ++i) {
        const int t = wsum[i];
        before += (i < w) ? t : 0;
        all += t;
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        off[e] = before + lower_lanes + mine;
        mine += pred[e] ? 1 : 0;
    }
    return all;
}

// Over `nbins` LDS bins taken from the top, find the bin holding the
// `need`-th largest item; returns the bin and the count strictly above it.
__device__ __forceinline__ void find_crossing(const uint32_t* bins, int nbins, int need, int* wsum,
                                              uint32_t* bc) {
    const int per = nbins / kFinishThreads;   // bins per thread, taken in descending order
    const int top = nbins - 1 - per * (int)threadIdx.x;
    int local = 0;
    for (int q = 0; q < per; ++q) local += (int)bins[top - q];
    int total;
    int c = wg_exclusive_scan(local, wsum, &total);
    for (int q = 0; q < per; ++q) {
        const int hcount = (int)bins[top - q];
        if (c < need && c + hcount >= need) {
            bc[0] = (uint32_t)(top - q);
            bc[1] = (uint32_t)c;
        }
        c += hcount;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kFinishThreads) sel_finish_kernel(const SelectArgs a) {
    __shared__ uint32_t bins[kSelBins];
    __shared__ int wsum[2][kFinishWaves];
    __shared__ uint32_t bc[2];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int seq0 = a.cu_seqlens_k[b];
    const int L = a.cu_seqlens_k[b + 1] - seq0 - a.W;
    const int kout = a.cu_k[b];
    const int k = min(a.cu_k[b + 1] - kout, L);
    if (k <= 0) return;
    int32_t* out = a.indices + kout;

    // a. top digit holding the k-th largest key.
    for (int i = tid; i < kSelBins; i += kFinishThreads) bins[i] = a.hist[(size_t)b * kSelBins + i];
    __syncthreads();
    find_crossing(bins, kSelBins, k, wsum[0], bc);
    const uint32_t d1 = bc[0];
    int above = (int)bc[1];

    // b. ordered compaction of positions whose top digit is >= d1.
    const uint32_t* keys = a.keys + seq0;
    int32_t* tpos = a.tmp_pos + seq0;
    uint32_t* tkey = a.tmp_key + seq0;
    int nsup = 0;
    int parity = 0;
    for (int base = 0; base < L; base += kRound) {
        const int p = base + kPer * tid;
        uint32_t kk[kPer];
        bool pred[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const bool in = (p + e) < L;
            kk[e] = in ? keys[p + e] : 0u;
            pred[e] = in && ((kk[e] >> (32 - kSelDigitBits)) >= d1);
        }
        int off[kPer];
        const int tot = round_offsets(pred, off, wsum[parity]);
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (pred[e]) {
                tpos[nsup + off[e]] = p + e;
                tkey[nsup + off[e]] = kk[e];
            }
        nsup += tot;
        parity ^= 1;
    }
    __syncthreads();   // scratch list complete and visible to the whole workgroup

    // c. refine: two 10-bit digits below the top digit.
    uint32_t prefix = d1;
    int need = k - above;
#pragma unroll 1
    for (int level = 0; level < 2; ++level) {
        const int shift = (level == 0) ? 10 : 0;
        const int pshift = shift + 10;
        for (int i = tid; i < 1024; i += kFinishThreads) bins[i] = 0u;
        __syncthreads();
        for (int i = tid; i < nsup; i += kFinishThreads) {
            const uint32_t key = tkey[i];
            if ((key >> pshift) == prefix) atomicAdd(&bins[(key >> shift) & 1023u], 1u);
        }
        __syncthreads();
        find_crossing(bins, 1024, need, wsum[0], bc);
        prefix = (prefix << 10) | bc[0];
        need -= (int)bc[1];
        above += (int)bc[1];
        __syncthreads();
    }
    const uint32_t theta = prefix;     // exact k-th largest key
    const int take_ties = need;        // positions equal to theta still to take (>= 1)

    // d. ordered compaction of the scratch list into T.
    int ties_seen = 0, written = 0;
    for (int base = 0; base < nsup; base += kRound) {
        const int i0 = base + kPer * tid;
        uint32_t kk[kPer];
        int32_t pp[kPer];
        bool tie[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const bool in = (i0 + e) < nsup;
            kk[e] = in ? tkey[i0 + e] : 0u;
            pp[e] = in ? tpos[i0 + e] : 0;
            tie[e] = in && kk[e] == theta;
        }
        int toff[kPer];
        const int ntie = round_offsets(tie, toff, wsum[parity]);
        parity ^= 1;
        bool sel[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const bool in = (i0 + e) < nsup;
            sel[e] = in && (kk[e] > theta || (tie[e] && ties_seen + toff[e] < take_ties));
        }
        int soff[kPer];
        const int nsel = round_offsets(sel, soff, wsum[parity]);
        parity ^= 1;
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            if (sel[e] && written + soff[e] < k) out[written + soff[e]] = pp[e];
        ties_seen += ntie;
        written += nsel;
    }
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
    const int nh = a.batch * kSelBins;
    hipLaunchKernelGGL(sel_zero_kernel, dim3((nh + 255) / 256), dim3(256), 0, stream, a.hist, nh);
    if (a.nchunks > 0)
        hipLaunchKernelGGL(sel_keys_kernel, dim3(a.nchunks, a.batch), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(sel_finish_kernel, dim3(a.batch), dim3(kFinishThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace vegas
