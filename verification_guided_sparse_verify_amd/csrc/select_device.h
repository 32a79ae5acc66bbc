// Device helpers of the exact top-k selection shared by the selection kernels
// and by the fused verification + selection path (whose combine kernel also
// does the selection's first step).  Included by .hip sources only.
#pragma once

#include "internal.h"

namespace vegas {
namespace {

__device__ __forceinline__ uint32_t order_key(float f) {
    f = f + 0.0f;                             // -0 and +0 share one key
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Clamped geometry of sequence b: first row, candidate count L (prefix), k
// and the first output slot.
struct SeqGeo {
    int seq0, L, k, kout;
};
__device__ __forceinline__ SeqGeo seq_geo(const SelectArgs& a, int b) {
    SeqGeo s;
    if (a.hg_n > 0) {                         // computed on the host from host copies of the offsets
        s.seq0 = a.hg_seq0[b];
        s.L = a.hg_L[b];
        s.k = a.hg_k[b];
        s.kout = a.hg_kout[b];
        return s;
    }
    s.seq0 = min(max(a.cu_seqlens_k[b], 0), a.total_kv);
    const int end = min(max(a.cu_seqlens_k[b + 1], s.seq0), a.total_kv);
    s.L = max(end - s.seq0 - a.W, 0);
    s.L = min(s.L, a.nchunks * kSelChunk);
    const int kend = max(a.cu_k[a.batch], 0);
    s.kout = min(max(a.cu_k[b], 0), kend);
    s.k = min(min(max(a.cu_k[b + 1] - s.kout, 0), s.L), kend - s.kout);
    return s;
}

// First selection step for one 2048-position chunk of sequence b: the
// per-position score summed over KV heads, its order-preserving key (stored),
// and the chunk's 12-bit top-digit histogram added into the sequence's
// histogram in a.zeroed (which must hold zeros before the first chunk).
// h: kSelBins words of LDS.  Called by whole workgroups of kSelThreads
// threads; returns with h free for reuse.
__device__ __forceinline__ void sel_keys_chunk(const SelectArgs& a, int b, int chunk, uint32_t* h) {
    const SeqGeo sg = seq_geo(a, b);
    const int start = chunk * kSelChunk;
    if (start >= sg.L) return;                         // uniform per workgroup
    for (int i = threadIdx.x; i < kSelBins; i += kSelThreads) h[i] = 0u;

    float s[kSelPer];
    bool in[kSelPer];
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        in[e] = start + e * kSelThreads + (int)threadIdx.x < sg.L;
        s[e] = 0.f;
    }
    const float* col = a.scores + sg.seq0 + start + threadIdx.x;
    // S = sum over KV heads 0, 1, ... in this order; eight heads' loads in flight.
    for (int g0 = 0; g0 < a.hkv; g0 += 8) {
        float x[8][kSelPer];
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
            const float* row = col + (size_t)(g0 + gi) * a.total_kv;
#pragma unroll
            for (int e = 0; e < kSelPer; ++e) x[gi][e] = (in[e] && g0 + gi < a.hkv) ? row[e * kSelThreads] : 0.f;
        }
#pragma unroll
        for (int gi = 0; gi < 8; ++gi)
#pragma unroll
            for (int e = 0; e < kSelPer; ++e)
                if (g0 + gi < a.hkv) s[e] += x[gi][e];
    }
    __syncthreads();                                   // histogram cleared
    uint32_t* keys = a.keys + sg.seq0 + start + threadIdx.x;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
        if (!in[e]) continue;
        const uint32_t key = order_key(s[e]);
        keys[e * kSelThreads] = key;
        atomicAdd(&h[key >> (32 - kSelDigitBits)], 1u);
    }
    __syncthreads();
    uint32_t* gh = a.zeroed + (size_t)b * kSelBins;
    for (int i = threadIdx.x; i < kSelBins; i += kSelThreads)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    __syncthreads();                                   // h is free again
}

}  // namespace
}  // namespace vegas
