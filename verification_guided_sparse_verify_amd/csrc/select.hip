// Exact top-k KV selection for gfx950.
//
// The selected set (gist.science "Technical Summary" of Vegas, sec. 2A
// "Formulation") is the size-k subset of the prefix maximising the collected
// logits summed over rows and query heads; for a sum of per-position terms it
// is the k positions with the largest per-position sum.  The verification
// kernel leaves one fp32 sum per (KV head, position); here
// S[i] = sum over KV heads, then an exact radix select on the
// order-preserving 32-bit image ("key") of S.
//
// Four launches, the last three spread over one workgroup per 2048-position
// chunk so that a long sequence is never left to a handful of compute units.
// Workgroups exchange results only across launch boundaries (on a multi-die
// part an in-kernel hand-off would need an L2 write-back per workgroup).
//   zero      clear the per-sequence histograms and candidate counters;
//   keys      S, its key, a 12-bit top-digit histogram (LDS, merged into the
//             per-sequence histogram with global atomics);
//   cand      every chunk finds the top digit d1 holding the k-th largest
//             key, counts its keys above d1 and appends the keys in bin d1
//             (the only undecided ones, typically ~1% of the prefix) to a
//             per-sequence candidate list;
//   write     every chunk recomputes, from the candidates, the exact k-th
//             largest key theta (two 10-bit refinement histograms), how many
//             keys equal to theta are taken (lowest positions first), and
//             the output offset and tie share of each chunk before it; then
//             writes its selected positions in ascending order at its offset.
// In the one-call verification + selection the verification kernels do zero
// (split kernel) and keys (combine kernel), and only cand and write launch
// here (launch_select_tail).
#include "internal.h"
#include "select_device.h"

namespace vegas {
namespace {

__global__ void sel_zero_kernel(uint32_t* __restrict__ p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Exclusive prefix sum of x over the workgroup's threads, in thread order;
// *total receives the sum.  wsum: kSelThreads/64 ints of LDS.
__device__ __forceinline__ int wg_exclusive_scan(int x, int* wsum, int* total) {
    constexpr int NW = kSelThreads / 64;
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
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int t = wsum[i];
        before += (i < w) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + v - x;
}

// Sum of x over the workgroup's threads (any order: integers); all threads get it.
__device__ __forceinline__ uint64_t wg_total(uint64_t x, uint64_t* wsum) {
    constexpr int NW = kSelThreads / 64;
    static_assert(kSelChunk < (1 << 16), "per-chunk counts are packed into 16 bits");
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = x;
    __syncthreads();
    uint64_t all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) all += wsum[i];
    __syncthreads();
    return all;
}

// Over NBINS LDS bins taken from the top, find the bin holding the
// `need`-th largest item (1 <= need <= sum of bins): out[0] = bin,
// out[1] = count of items in bins strictly above it.
template <int NBINS>
__device__ __forceinline__ void find_crossing(const uint32_t* bins, int need, int* wsum, uint32_t* out) {
    constexpr int PER = NBINS / kSelThreads;  // bins per thread, taken in descending order
    const int top = NBINS - 1 - PER * (int)threadIdx.x;
    uint32_t h[PER];
    int local = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        h[q] = bins[top - q];
        local += (int)h[q];
    }
    int total;
    int c = wg_exclusive_scan(local, wsum, &total);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int hcount = (int)h[q];
        if (c < need && c + hcount >= need) {
            out[0] = (uint32_t)(top - q);
            out[1] = (uint32_t)c;
        }
        c += hcount;
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kSelThreads) sel_keys_kernel(const SelectArgs a) {
    __shared__ uint32_t h[kSelBins];
    sel_keys_chunk(a, blockIdx.y, blockIdx.x, h);
}

__global__ void __launch_bounds__(kSelThreads) sel_cand_kernel(const SelectArgs a) {
    __shared__ uint32_t bins[kSelBins];
    __shared__ int wsum[kSelThreads / 64];
    __shared__ uint32_t cross[2];
    __shared__ uint32_t base_s;
    const int b = blockIdx.y;
    const int chunk = blockIdx.x;
    const SeqGeo sg = seq_geo(a, b);
    const int start = chunk * kSelChunk;
    if (sg.k <= 0 || start >= sg.L) return;            // uniform per workgroup

    // This chunk's keys (in flight while the histogram is scanned).
    const uint32_t* keys = a.keys + sg.seq0 + start + threadIdx.x;
    uint32_t kk[kSelPer];
    bool in[kSelPer];
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        in[e] = start + e * kSelThreads + (int)threadIdx.x < sg.L;
        kk[e] = in[e] ? keys[e * kSelThreads] : 0u;
    }
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.zeroed + (size_t)b * kSelBins);
        uint4 h4[kSelBins / 4 / kSelThreads];
#pragma unroll
        for (int q = 0; q < kSelBins / 4 / kSelThreads; ++q) h4[q] = src[q * kSelThreads + threadIdx.x];
#pragma unroll
        for (int q = 0; q < kSelBins / 4 / kSelThreads; ++q)
            reinterpret_cast<uint4*>(bins)[q * kSelThreads + threadIdx.x] = h4[q];
    }
    __syncthreads();
    find_crossing<kSelBins>(bins, sg.k, wsum, cross);
    const uint32_t d1 = cross[0];
    if (chunk == 0 && threadIdx.x == 0) {
        a.seq_info[4 * b + 0] = d1;
        a.seq_info[4 * b + 1] = cross[1];
    }

    bool cand[kSelPer];
    int above = 0, ncand = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        const uint32_t dig = kk[e] >> (32 - kSelDigitBits);
        above += (in[e] && dig > d1) ? 1 : 0;
        cand[e] = in[e] && dig == d1;
        ncand += cand[e] ? 1 : 0;
    }
    // One counter update per workgroup; candidate order does not matter.
    int total;
    int off = wg_exclusive_scan(ncand, wsum, &total);
    if (threadIdx.x == 0)
        base_s = total ? atomicAdd(&a.zeroed[(size_t)a.batch * kSelBins + b], (uint32_t)total) : 0u;
    int above_all;
    wg_exclusive_scan(above, wsum, &above_all);        // also orders base_s before the reads
    const uint32_t base = base_s;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        if (!cand[e]) continue;
        const int slot = (int)base + off++;
        if (slot < sg.L) {
            a.cand_key[sg.seq0 + slot] = kk[e];
            a.cand_pos[sg.seq0 + slot] = start + e * kSelThreads + (int)threadIdx.x;
        }
    }
    if (threadIdx.x == 0) a.chunk_above[(size_t)b * a.nchunks + chunk] = (uint32_t)above_all;
}

__global__ void __launch_bounds__(kSelThreads) sel_write_kernel(const SelectArgs a) {
    __shared__ uint32_t bins[1024];
    // Per-chunk counts of candidates above and equal to theta (a.nchunks each,
    // sized at launch: small enough to share a CU with a verification workgroup).
    extern __shared__ uint32_t sel_dyn[];
    uint32_t* gt = sel_dyn;
    uint32_t* ties = sel_dyn + a.nchunks;
    __shared__ int wsum[kSelThreads / 64];
    __shared__ uint64_t wsum64[kSelThreads / 64];
    __shared__ uint32_t cross[2];
    const int b = blockIdx.y;
    const int chunk = blockIdx.x;
    const int tid = threadIdx.x;
    const SeqGeo sg = seq_geo(a, b);
    const int start = chunk * kSelChunk;
    if (sg.k <= 0 || start >= sg.L) return;            // uniform per workgroup

    // This chunk's keys: thread t owns the consecutive positions start + kSelPer*t + e.
    const int p0 = start + kSelPer * tid;
    uint32_t kk[kSelPer];
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) kk[e] = (p0 + e < sg.L) ? a.keys[sg.seq0 + p0 + e] : 0u;

    const uint32_t d1 = a.seq_info[4 * b + 0];
    const int above1 = (int)a.seq_info[4 * b + 1];
    const int nc = min((int)a.zeroed[(size_t)a.batch * kSelBins + b], sg.L);
    const uint32_t* ck = a.cand_key + sg.seq0;
    const int32_t* cp = a.cand_pos + sg.seq0;
    const int nch = min((sg.L + kSelChunk - 1) / kSelChunk, a.nchunks);

    // Candidates: the first kSelThreads*kCandPer stay in registers for all
    // passes (typically all of them); any beyond are re-read per pass.
    constexpr int kCandPer = 8;
    constexpr int kCandHeld = kSelThreads * kCandPer;
    uint32_t hk[kCandPer];
    int32_t hp[kCandPer];
#pragma unroll
    for (int e = 0; e < kCandPer; ++e) {
        const int i = e * kSelThreads + tid;
        hk[e] = ck[min(i, sg.L - 1)];        // issued with the count's load; slots >= nc unused
        hp[e] = cp[min(i, sg.L - 1)];
    }
    // Keys above the top digit in the chunks before this one (loaded up front).
    int above_before = 0;
    for (int c = tid; c < chunk; c += kSelThreads) above_before += (int)a.chunk_above[(size_t)b * a.nchunks + c];
    // Visit every candidate (key, position) once: held ones first, then the rest
    // in batches of kCandPer loads per thread.
    auto for_each_cand = [&](auto&& fn) {
#pragma unroll
        for (int e = 0; e < kCandPer; ++e)
            if (e * kSelThreads + tid < nc) fn(hk[e], hp[e]);
        for (int base = kCandHeld; base < nc; base += kCandHeld) {
            uint32_t bk[kCandPer];
            int32_t bp[kCandPer];
#pragma unroll
            for (int e = 0; e < kCandPer; ++e) {
                const int i = base + e * kSelThreads + tid;
                bk[e] = i < nc ? ck[i] : 0u;
                bp[e] = i < nc ? cp[i] : 0;
            }
#pragma unroll
            for (int e = 0; e < kCandPer; ++e)
                if (base + e * kSelThreads + tid < nc) fn(bk[e], bp[e]);
        }
    };

    // Exact theta: two 10-bit digits below the top digit, over the candidates.
    uint32_t prefix = d1;
    int need = sg.k - above1;                 // keys of bin d1 still to take, >= 1
#pragma unroll 1
    for (int level = 0; level < 2; ++level) {
        const int shift = level == 0 ? 10 : 0;
        for (int i = tid; i < 1024; i += kSelThreads) bins[i] = 0u;
        __syncthreads();
        for_each_cand([&](uint32_t key, int32_t) {
            if ((key >> (shift + 10)) == prefix) atomicAdd(&bins[(key >> shift) & 1023u], 1u);
        });
        __syncthreads();
        find_crossing<1024>(bins, need, wsum, cross);
        prefix = (prefix << 10) | cross[0];
        need -= (int)cross[1];
        __syncthreads();
    }
    const uint32_t theta = prefix;            // the k-th largest key
    const int take = need;                    // keys equal to theta to take, lowest positions first

    // Chunks up to this one: candidates above theta and equal to theta.
    for (int c = tid; c <= chunk; c += kSelThreads) {
        gt[c] = 0u;
        ties[c] = 0u;
    }
    __syncthreads();
    for_each_cand([&](uint32_t key, int32_t pos) {
        const int c = min(max(pos, 0) >> kSelChunkShift, nch - 1);
        if (c <= chunk) {
            if (key > theta) atomicAdd(&gt[c], 1u);
            else if (key == theta) atomicAdd(&ties[c], 1u);
        }
    });
    __syncthreads();
    // Output offset of this chunk and its tie share, from the chunks before it.
    // Both totals in one reduction: ties in the low word, keys above theta in
    // the high word (each below 2^31).
    uint32_t tl = 0, sl = (uint32_t)above_before;
    for (int c = tid; c < chunk; c += kSelThreads) {
        tl += ties[c];
        sl += gt[c];
    }
    const uint64_t both = wg_total(((uint64_t)sl << 32) | tl, wsum64);
    const int ties_before = (int)(uint32_t)both;
    const int sel_before = (int)(both >> 32);
    const int off0 = sel_before + min(ties_before, take);
    const int tq = min(max(take - ties_before, 0), (int)ties[chunk]);

    bool gtp[kSelPer], tie[kSelPer];
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        const bool in = p0 + e < sg.L;
        gtp[e] = in && kk[e] > theta;
        tie[e] = in && kk[e] == theta;
    }
    // One scan gives, for every item, the keys above theta and the ties before
    // it (packed 16/16: a chunk holds at most kSelChunk of each).  The ties
    // taken are the first tq in position order, so an item's output slot is
    // (above theta before it) + min(ties before it, tq).
    int mine = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) mine += (gtp[e] ? 1 << 16 : 0) + (tie[e] ? 1 : 0);
    int total;
    int before = wg_exclusive_scan(mine, wsum, &total);
    int32_t* out = a.indices + sg.kout;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        const int gb = before >> 16, tb = before & 0xFFFF;
        const bool sel = gtp[e] || (tie[e] && tb < tq);
        const int slot = off0 + gb + min(tb, tq);
        if (sel && slot >= 0 && slot < sg.k) out[slot] = p0 + e;
        before += (gtp[e] ? 1 << 16 : 0) + (tie[e] ? 1 : 0);
    }
}

// One thread per output slot: find the slot's sequence (binary search over
// cu_idx), then emit sink j (j < min(sinks, k)) or recent position L-(k-j).
__global__ void streaming_indices_kernel(int batch, int W, int sinks, const int32_t* __restrict__ cu_seqlens_k,
                                         int32_t total_kv, const int32_t* __restrict__ cu_idx, int32_t total_idx,
                                         int32_t* __restrict__ indices) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_idx) return;
    int lo = 0, hi = batch;                   // sequence b with cu_idx[b] <= i < cu_idx[b+1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu_idx[mid] <= i) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int s0 = min(max(cu_seqlens_k[b], 0), total_kv);
    const int L = max(min(max(cu_seqlens_k[b + 1], s0), total_kv) - s0 - W, 0);
    const int k = min(cu_idx[b + 1] - cu_idx[b], L);
    const int j = i - cu_idx[b];
    const int ns = min(sinks, k);
    int pos = j < ns ? j : L - (k - j);
    indices[i] = min(max(pos, 0), max(L - 1, 0));
}

}  // namespace

hipError_t launch_streaming_indices(int batch, int W, int sinks, const int32_t* cu_seqlens_k, int32_t total_kv,
                                    const int32_t* cu_idx, int32_t total_idx, int32_t* indices,
                                    hipStream_t stream) {
    if (total_idx > 0)
        hipLaunchKernelGGL(streaming_indices_kernel, dim3((total_idx + 255) / 256), dim3(256), 0, stream, batch, W,
                           sinks, cu_seqlens_k, total_kv, cu_idx, total_idx, indices);
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
    const int nz = select_zeroed_words(a.batch);
    hipLaunchKernelGGL(sel_zero_kernel, dim3((nz + 1023) / 1024), dim3(256), 0, stream, a.zeroed, nz);
    if (a.nchunks > 0)
        hipLaunchKernelGGL(sel_keys_kernel, dim3(a.nchunks, a.batch), dim3(kSelThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_select_tail(a, stream);
}

hipError_t launch_select_from_keys(const SelectArgs& a, hipStream_t stream) {
    if (a.nchunks > 0)
        hipLaunchKernelGGL(sel_keys_kernel, dim3(a.nchunks, a.batch), dim3(kSelThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_select_tail(a, stream);
}

hipError_t launch_select_tail(const SelectArgs& a, hipStream_t stream) {
    if (a.nchunks > 0) {
        const dim3 grid(a.nchunks, a.batch);
        hipLaunchKernelGGL(sel_cand_kernel, grid, dim3(kSelThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_write_kernel, grid, dim3(kSelThreads), 2 * a.nchunks * sizeof(uint32_t), stream, a);
    }
    return hipGetLastError();
}

}  // namespace vegas
