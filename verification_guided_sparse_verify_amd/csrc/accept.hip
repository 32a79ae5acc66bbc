// Speculative-sampling acceptance for gfx950: the step that follows
// verification in self-speculative decoding (blog "You Could Have Come Up
// with Speculative Decoding", section "Preservation of Target Distribution").
// Draft token y_j, proposed from q_j, is kept when u_j * q_j(y_j) <= p_j(y_j);
// at the first rejection a replacement is drawn from max(0, p_j - q_j)
// normalised; when every draft is kept, the bonus token is drawn from
// p_{gamma+1}.
//
// Arithmetic that decides tokens is fixed so that the result does not depend
// on the order of any sum:
//   - the acceptance test is exact: a product of two binary32 values is exact
//     in binary64;
//   - masses are fixed point, m_y = floor(x_y * 2^40) (capped at 2^40) of the
//     residual or probability x_y, summed as 64-bit integers;
//   - the draw is the smallest y with m_0 + ... + m_y > floor(u24 * M / 2^24),
//     u24 = floor(u * 2^24), M = sum of all masses;
//   - a zero residual mass (rounding or unnormalised inputs) falls back to p_j,
//     and a zero mass there to token 0.
// Two launches over 4096-token chunks of the vocabulary (all coalesced):
//   mass   every chunk workgroup decides the first rejection j (lane j of one
//          wave tests draft j) and sums its chunk's residual and target masses;
//   draw   every chunk workgroup forms the totals and its prefix from the chunk
//          sums; the one holding the draw scans its chunk in order.
#include "internal.h"

namespace vegas {
namespace {

constexpr int kAccThreads = 256;
constexpr int kAccWaves = kAccThreads / 64;
constexpr int kAccPer = kAcceptChunk / kAccThreads;   // tokens per thread per chunk

__device__ __forceinline__ uint64_t fixed_mass(double x) {
    if (!(x > 0.0)) return 0;
    double f = floor(x * 1099511627776.0);        // 2^40
    if (f > 1099511627776.0) f = 1099511627776.0;
    return (uint64_t)f;
}

// Index of the first rejected draft (gamma if none); all threads get it.
__device__ __forceinline__ int first_rejection(int b, int gamma, int64_t vocab, const float* pb, const float* qb,
                                               const int32_t* draft, const float* u_accept, int* s) {
    if (threadIdx.x < 64) {
        bool rejected = false;
        const int j = threadIdx.x;
        if (j < gamma) {
            const int64_t y = min(max((int64_t)draft[(int64_t)b * gamma + j], (int64_t)0), vocab - 1);
            const double lhs = (double)u_accept[(int64_t)b * gamma + j] * (double)qb[(int64_t)j * vocab + y];
            rejected = !(lhs <= (double)pb[(int64_t)j * vocab + y]);
        }
        const uint64_t bal = __ballot(rejected);
        if (threadIdx.x == 0) *s = bal ? __ffsll((unsigned long long)bal) - 1 : gamma;
    }
    __syncthreads();
    return *s;
}

// Sum over the workgroup of two 64-bit values (exact, any order).
__device__ __forceinline__ void wg_sum2(uint64_t& a, uint64_t& b, uint64_t (*red)[2]) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
    }
    if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6][0] = a;
        red[threadIdx.x >> 6][1] = b;
    }
    __syncthreads();
    a = 0;
    b = 0;
#pragma unroll
    for (int w = 0; w < kAccWaves; ++w) {
        a += red[w][0];
        b += red[w][1];
    }
}

__global__ void __launch_bounds__(kAccThreads)
accept_mass_kernel(const AcceptArgs a) {
    __shared__ int j_s;
    __shared__ uint64_t red[kAccWaves][2];
    const int c = blockIdx.x;
    const int b = blockIdx.y;
    const float* pb = a.p + (int64_t)b * (a.gamma + 1) * a.vocab;
    const float* qb = a.gamma > 0 ? a.q + (int64_t)b * a.gamma * a.vocab : nullptr;
    const int j = first_rejection(b, a.gamma, a.vocab, pb, qb, a.draft, a.u_accept, &j_s);
    const float* prow = pb + (int64_t)j * a.vocab;
    const float* qrow = j < a.gamma ? qb + (int64_t)j * a.vocab : nullptr;
    uint64_t res = 0, tgt = 0;
    const int64_t y0 = (int64_t)c * kAcceptChunk;
#pragma unroll
    for (int e = 0; e < kAccPer; ++e) {
        const int64_t y = y0 + e * kAccThreads + threadIdx.x;
        if (y < a.vocab) {
            const double pv = (double)prow[y];
            tgt += fixed_mass(pv);
            res += qrow ? fixed_mass(pv - (double)qrow[y]) : 0;
        }
    }
    wg_sum2(res, tgt, red);
    if (threadIdx.x == 0) {
        uint64_t* part = a.part + ((size_t)b * a.nchunks + c) * 2;
        part[0] = res;
        part[1] = tgt;
        if (c == 0) a.first_rej[b] = j;
    }
}

__global__ void __launch_bounds__(kAccThreads)
accept_draw_kernel(const AcceptArgs a) {
    __shared__ uint64_t wsum[kAccWaves];
    __shared__ uint64_t red[kAccWaves][2];
    const int c = blockIdx.x;
    const int b = blockIdx.y;
    const int j = a.first_rej[b];
    const uint64_t* part = a.part + (size_t)b * a.nchunks * 2;
    // Totals and this chunk's prefix from the chunk sums (each thread a strided share).
    uint64_t tres = 0, ttgt = 0, bres = 0, btgt = 0;
    for (int i = threadIdx.x; i < a.nchunks; i += kAccThreads) {
        const uint64_t r = part[2 * i], t = part[2 * i + 1];
        tres += r;
        ttgt += t;
        if (i < c) {
            bres += r;
            btgt += t;
        }
    }
    wg_sum2(tres, ttgt, red);
    __syncthreads();
    wg_sum2(bres, btgt, red);
    const bool residual = j < a.gamma && tres > 0;
    const uint64_t total = residual ? tres : ttgt;
    if (total == 0) {                                 // nothing to draw from: token 0
        if (c == 0 && threadIdx.x == 0) {
            a.n_accepted[b] = j;
            a.next_token[b] = 0;
        }
        return;
    }
    const double uf = floor((double)a.u_sample[b] * 16777216.0);   // 2^24
    const uint64_t ui = uf < 0.0 ? 0 : (uf > 16777215.0 ? 16777215u : (uint64_t)uf);
    const uint64_t thr = (total >> 24) * ui + (((total & 16777215u) * ui) >> 24);
    const uint64_t before_chunk = residual ? bres : btgt;
    if (c == 0 && threadIdx.x == 0) a.n_accepted[b] = j;
    __syncthreads();
    // Only the chunk whose mass range holds thr goes on (uniform per workgroup).
    const uint64_t chunk_mass = residual ? part[2 * c] : part[2 * c + 1];
    if (!(before_chunk <= thr && thr < before_chunk + chunk_mass)) return;

    const float* prow = a.p + ((int64_t)b * (a.gamma + 1) + j) * a.vocab;
    const float* qrow = residual ? a.q + ((int64_t)b * a.gamma + j) * a.vocab : nullptr;
    // Thread t owns the consecutive tokens y0 + kAccPer*t + e.
    const int64_t y0 = (int64_t)c * kAcceptChunk + (int64_t)kAccPer * threadIdx.x;
    uint64_t m[kAccPer];
    uint64_t mine = 0;
#pragma unroll
    for (int e = 0; e < kAccPer; ++e) {
        const int64_t y = y0 + e;
        m[e] = 0;
        if (y < a.vocab) {
            const double pv = (double)prow[y];
            m[e] = qrow ? fixed_mass(pv - (double)qrow[y]) : fixed_mass(pv);
        }
        mine += m[e];
    }
    // Exclusive scan of the per-thread masses in thread order.
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    uint64_t v = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = __shfl_up(v, off);
        if (lane >= off) v += y;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    uint64_t run = before_chunk + v - mine;
    for (int i = 0; i < w; ++i) run += wsum[i];
    if (run <= thr && thr < run + mine) {            // exactly one thread
#pragma unroll
        for (int e = 0; e < kAccPer; ++e) {
            run += m[e];
            if (run > thr) {
                a.next_token[b] = (int32_t)(y0 + e);
                break;
            }
        }
    }
}

}  // namespace

hipError_t launch_spec_accept(const AcceptArgs& a, hipStream_t stream) {
    if (a.batch > 0 && a.nchunks > 0) {
        const dim3 grid(a.nchunks, a.batch);
        hipLaunchKernelGGL(accept_mass_kernel, grid, dim3(kAccThreads), 0, stream, a);
        hipLaunchKernelGGL(accept_draw_kernel, grid, dim3(kAccThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace vegas
