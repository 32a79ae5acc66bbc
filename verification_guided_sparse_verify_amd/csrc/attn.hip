// Split-K attention for gfx950: the verification pass and the sparse drafting
// pass of Vegas share this kernel.
//
// Verification ("Vegas ...", sec. 4 "Attention kernel implementation"): the
// gamma+1 new rows of every query head attend to the whole KV cache with a
// bottom-right causal mask, and the pre-softmax logits of the collected rows
// (Collect-2-Query, sec. 3.3) are summed over the query heads of each KV head
// and written to HBM.  Drafting (sec. 4 "Serving framework integration"): one
// query row per head attends to a list of token positions (pages of one
// token).
//
// Work decomposition.  A workgroup owns one (sequence b, KV head g, position
// split); the host sizes splits so that the grid is one round of workgroups
// on the 256 CUs.  All W*G query rows that share KV head g (at most 64) are
// processed together, so every K/V byte is read from HBM exactly once for all
// rows.  The four waves take 16-position blocks in turn; each wave streams its
// blocks through a private two-stage LDS ring filled by the load-to-LDS path
// (no VGPR round trip), computing one block while the next is in flight.
// A wave holds all the row tiles (up to four).  Per block and wave:
//   S^T[pos, row] = K[pos, :] . Q[row, :]          16x16x32 bf16 MFMA; K from
//                                                   the ring, Q in registers
//   collection (verification only)                 collected rows summed over
//                                                   the query heads of g: a
//                                                   16-lane DPP butterfly,
//                                                   buffered in LDS
//   online softmax over positions (exp2 domain)    rows are MFMA columns, so a
//                                                   row max is in-lane + 2 shuffles
//   O^T[d, row] += V^T[d, pos] . P^T[pos, row]     16x16x16 bf16 MFMA; V^T read
//                                                   transposed from the ring
// The P^T operand is the S^T accumulator itself: the k order of an MFMA is a
// free permutation, so the four S^T values a lane owns are exactly its four k
// slots, and V^T is read in that order.  Partials (m, l, O) of the four waves
// are merged in LDS and one partial per workgroup goes to the workspace; the
// collected scores of the split are written with coalesced stores;
// attn_combine merges the splits (and, in the one-call verification +
// selection, also runs the selection's first step).
#include "internal.h"
#include "select_device.h"

namespace vegas {

#ifdef VEGAS_PHASE_TRACE
// Measurement build only (libvegas_trace.so, never the product library):
// each split workgroup records its start, the end of its last unit's block
// loop and its end (the 100 MHz constant clock), the hardware ids of the CU
// it ran on and its (sequence, split, KV head); vegas_trace_read copies the
// records out.  g_trace_rotate != 0 maps workgroup w to KV head
// (w + w / Hkv) % Hkv instead of w % Hkv, so a KV head's workgroups land on
// every XCD (the dispatcher deals workgroups to the XCDs in turn).
constexpr int kTraceMax = 4096;
__device__ unsigned long long g_trace[kTraceMax][8];
__device__ unsigned long long g_trace_loop[kTraceMax];
__device__ int g_trace_rotate;
#endif

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr float kNegInf = -__builtin_inff();

// Eight operand elements owned by one lane.
template <bool BF16> struct Frag;
template <> struct Frag<true> { uint4 u; };
template <> struct Frag<false> { uint4 u[2]; };

template <bool BF16>
__device__ __forceinline__ Frag<BF16> zero_frag() {
    Frag<BF16> r;
    if constexpr (BF16) {
        r.u = make_uint4(0, 0, 0, 0);
    } else {
        r.u[0] = make_uint4(0, 0, 0, 0);
        r.u[1] = make_uint4(0, 0, 0, 0);
    }
    return r;
}

// p points at 8 consecutive elements (16 B for bf16, 32 B for fp32), 16-B aligned.
template <bool BF16>
__device__ __forceinline__ Frag<BF16> load_frag(const void* p) {
    Frag<BF16> r;
    if constexpr (BF16) {
        r.u = *reinterpret_cast<const uint4*>(p);
    } else {
        r.u[0] = reinterpret_cast<const uint4*>(p)[0];
        r.u[1] = reinterpret_cast<const uint4*>(p)[1];
    }
    return r;
}

// acc += A(16 x 32) * B(32 x 16).  Lane l supplies row/column l%16 and the
// eight k slots 8*(l/16) .. 8*(l/16)+7; fp32 runs the same contraction as
// eight k=4 MFMAs, slot m of every lane forming the m-th one.
__device__ __forceinline__ f32x4_t mfma16(const Frag<true>& a, const Frag<true>& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                   __builtin_bit_cast(bf16x8_t, b.u), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(const Frag<false>& a, const Frag<false>& b, f32x4_t c) {
    const uint32_t xs[8] = {a.u[0].x, a.u[0].y, a.u[0].z, a.u[0].w, a.u[1].x, a.u[1].y, a.u[1].z, a.u[1].w};
    const uint32_t ys[8] = {b.u[0].x, b.u[0].y, b.u[0].z, b.u[0].w, b.u[1].x, b.u[1].y, b.u[1].z, b.u[1].w};
#pragma unroll
    for (int m = 0; m < 8; ++m)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(xs[m]), __uint_as_float(ys[m]), c, 0, 0, 0);
    return c;
}

template <bool BF16>
__device__ __forceinline__ Frag<BF16> pack_probs(const float (&p)[8]) {
    Frag<BF16> r;
    if constexpr (BF16) {
        bf16x8_t v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<__bf16>(p[i]);
        r.u = __builtin_bit_cast(uint4, v);
    } else {
        r.u[0] = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]),
                            __float_as_uint(p[3]));
        r.u[1] = make_uint4(__float_as_uint(p[4]), __float_as_uint(p[5]), __float_as_uint(p[6]),
                            __float_as_uint(p[7]));
    }
    return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}

// Four sums over the 16 lanes of a DPP row at once, scattered: lane r of the
// row returns the sum of x[r / 4] over the row.  Each step halves the values a
// lane carries: lanes r and r^8 (row_ror 8) swap halves of their four, lanes r
// and 7-r within each half row (row_half_mirror; they differ in bit 2 and
// share bit 3) swap halves of the remaining two, then the pairs r^1 and r^2
// (quad permutations) finish the single value: 5 DPP adds instead of 16.
__device__ __forceinline__ float row16_sum4(const float (&x)[4], int lr) {
    const bool b3 = (lr & 8) != 0, b2 = (lr & 4) != 0;
    const float y0 = (b3 ? x[2] : x[0]) + dpp<0x128>(b3 ? x[0] : x[2]);
    const float y1 = (b3 ? x[3] : x[1]) + dpp<0x128>(b3 ? x[1] : x[3]);
    float z = (b2 ? y1 : y0) + dpp<0x141>(b2 ? y0 : y1);
    z += dpp<0xB1>(z);   // quad_perm [1,0,3,2]
    z += dpp<0x4E>(z);   // quad_perm [2,3,0,1]
    return z;
}

// Max and sum over the lane pairs (l, l^16) and (l, l^32): gfx950's permlane
// swaps leave the pair's two values in the two outputs (checked on the device
// with a probe), a VALU exchange where a shuffle would go through LDS.
__device__ __forceinline__ float pair16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Compiler barrier that also drains outstanding LDS operations of this wave.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One wave-wide 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes land at
// lds + 16*l.  Issued as inline assembly on purpose: the compiler's wait
// analysis would otherwise make every later LDS read wait for all copies in
// flight, including the next block's.  Completion is ordered by vmcnt like
// any load, and the block loop waits for it explicitly (wait_vmem).
// The copy carries the non-temporal cache policy (nt): every K/V row is read
// once per call, and streaming reads with that policy run at ~7.2 TB/s on
// MI355X against ~6.3 TB/s with the default one (same kernel otherwise).
__device__ __forceinline__ void copy16_to_lds(const void* src, unsigned char* lds) {
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds_addr) : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they retire in issue order); also a compiler memory barrier.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Make the compiler treat a fragment as consumed here (it then waits for the
// load that produced it at this point).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void keep_live(uint4& u) {
    u32x4_t t = __builtin_bit_cast(u32x4_t, u);
    asm volatile("" : "+v"(t));
    u = __builtin_bit_cast(uint4, t);
}
__device__ __forceinline__ void keep_live(Frag<true>& f) { keep_live(f.u); }
__device__ __forceinline__ void keep_live(Frag<false>& f) {
    keep_live(f.u[0]);
    keep_live(f.u[1]);
}

template <bool BF16, int D, int MB, bool GATHER>
struct Geo {
    static constexpr int ES = BF16 ? 2 : 4;       // element bytes
    static constexpr int DC = D / 32;             // k chunks of the QK^T contraction
    static constexpr int DB = D / 16;             // 16-wide d tiles of the PV product
    static constexpr int ROWB = D * ES;           // bytes of one K/V row of one head
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static constexpr int EPC = 16 / ES;           // elements per chunk
    static constexpr int RPI = 64 / CPR;          // rows covered by one wave-wide 16-B copy
    static constexpr int TLD = kAttnBlock / RPI;  // copies per lane per K (or V) tile
    static constexpr int TILE = kAttnBlock * ROWB;
    static constexpr int STAGE = 2 * TILE;        // K tile then V tile
    static constexpr int NST = attn_stages(BF16, D, GATHER);   // ring depth
    static constexpr int RING = kAttnWaves * NST * STAGE;
    static constexpr int BLOCK_OPS = 2 * TLD;     // copies one block issues
    static constexpr int SWZU = 16 / EPC;         // chunks per 16-element d tile
    static constexpr int KSWZ = CPR - 1 < 15 ? CPR - 1 : 15;
    static constexpr int NREG = DB * MB;          // O^T fragments per lane
    static constexpr int MSLOT = (NREG * 4 + 2 * MB) * 64 * 4;
    static constexpr int MAIN = RING > (kAttnWaves / 2) * MSLOT ? RING : (kAttnWaves / 2) * MSLOT;
};

// Per-workgroup constants of the split kernel.  Offsets are 32-bit byte
// offsets from the first token row of the sequence (the host bounds them).
struct SplitCtx {
    const unsigned char* kbase;   // contiguous: the sequence's first K row; paged: the page pool
    const unsigned char* vbase;
    const int* idx_s;     // gather: staged rows of this split (positions, or pool rows if paged)
    const int* page_s;    // paged verification: pool pages of the split's positions
    int page0;            // paged verification: first page of the split
    int page_shift;       // log2(page size), or -1 for a contiguous cache
    int row_stride;       // bytes per token row: Hkv * D * element size
    int head_off;         // g * D * element size
    int start, end;       // position range of this split
};

// Byte offset from kbase/vbase of the row of position p (clamped into the split).
template <bool GATHER>
__device__ __forceinline__ uint64_t row_offset(const SplitCtx& c, int p) {
    const int pc = min(p, c.end - 1);
    uint32_t row;
    if constexpr (GATHER) {
        row = (uint32_t)c.idx_s[pc - c.start];
    } else if (c.page_shift >= 0) {
        const uint32_t page = (uint32_t)c.page_s[(pc >> c.page_shift) - c.page0];
        row = (page << c.page_shift) | ((uint32_t)pc & ((1u << c.page_shift) - 1u));
    } else {
        row = (uint32_t)pc;
    }
    return (uint64_t)row * (uint32_t)c.row_stride + (uint32_t)c.head_off;
}

// Copy the K and V rows of the 16 positions from p0 into one ring stage.
// Copy i of a tile fills LDS bytes [1024*i, 1024*i+1024): lane l lands on
// row RPI*i + l/CPR at chunk position l%CPR, and fetches the global chunk the
// tile's swizzle puts there.  K chunks are XORed with the row (so the 16
// lanes reading one chunk column of 16 rows hit distinct banks); V chunks are
// XORed with the row's 4-row group (so the transposed reads, four lane groups
// on rows 4 apart, hit distinct banks).
template <class GEO, bool GATHER>
__device__ __forceinline__ void issue_block(const SplitCtx& c, int p0, int lane, unsigned char* stage) {
    // All row offsets first (in gather mode, LDS reads of the index list that
    // then complete together), then the copies back to back.
    uint64_t off[GEO::TLD];
#pragma unroll
    for (int i = 0; i < GEO::TLD; ++i) off[i] = row_offset<GATHER>(c, p0 + i * GEO::RPI + lane / GEO::CPR);
#pragma unroll
    for (int i = 0; i < GEO::TLD; ++i) {
        const int row = i * GEO::RPI + lane / GEO::CPR;
        const int cc = (lane % GEO::CPR) ^ (row & GEO::KSWZ);
        copy16_to_lds(c.kbase + off[i] + cc * 16, stage + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < GEO::TLD; ++i) {
        const int row = i * GEO::RPI + lane / GEO::CPR;
        const int cc = (lane % GEO::CPR) ^ (GEO::SWZU * ((row >> 2) & 3));
        copy16_to_lds(c.vbase + off[i] + cc * 16, stage + GEO::TILE + i * 1024);
    }
}

// Positions of sequence b that a pass covers: [lo, lo + len) of its rows for
// verification (lo > 0 only under a local mask), or its list for gathering.
struct SeqSpan {
    int seq0, n_b, L, lo, len, ib0;
};
template <bool GATHER>
__device__ __forceinline__ SeqSpan seq_span(const AttnArgs& a, int b) {
    SeqSpan s;
    s.seq0 = min(max(a.cu_seqlens_k[b], 0), a.total_kv);
    s.n_b = min(max(a.cu_seqlens_k[b + 1], s.seq0), a.total_kv) - s.seq0;
    s.ib0 = 0;
    if constexpr (GATHER) {
        s.ib0 = a.cu_idx[b];
        s.L = 0;
        s.lo = 0;
        s.len = s.n_b > 0 ? max(a.cu_idx[b + 1] - s.ib0, 0) : 0;
    } else {
        s.L = s.n_b - a.W;
        s.lo = a.window > 0 ? max(0, s.L - a.window + 1) : 0;
        s.len = max(s.n_b - s.lo, 0);
    }
    return s;
}

// Split plan of one sequence: a share of `target` splits (per KV head, for the
// whole batch) proportional to its positions, but no split longer than
// a.chunk_cap; split length a multiple of kAttnWaves*kAttnBlock.  Ragged
// batches so get about equal work per workgroup.  Integer arithmetic: every
// workgroup of a pass, and the host plan, evaluate it identically.
__device__ __forceinline__ void seq_plan(const AttnArgs& a, int len, int total, int target, int& ns, int& chunk) {
    constexpr int unit = kAttnWaves * kAttnBlock;
    if (len <= 0) {
        ns = 0;
        chunk = unit;
        return;
    }
    // ceil(len * target / total) in exact integer arithmetic (the host plan
    // evaluates the same expression)
    int want = (int)(((long long)len * target + total - 1) / total);
    want = max(max(want, 1), (len + a.chunk_cap - 1) / a.chunk_cap);
    chunk = (len + want - 1) / want;
    chunk = (chunk + unit - 1) / unit * unit;
    ns = min((len + chunk - 1) / chunk, a.nsplit);
}

// Sum of x over the NT threads of the workgroup (all get it).  red: NT/64 ints of LDS.
template <int NT>
__device__ __forceinline__ int wg_sum(int x, int* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += red[w];
    return t;
}

// The batch's split plan as every workgroup of a pass sees it.  Thread t holds
// sequences t, t + blockDim, ... (at most kPlanPerThread of them).  The split
// target is the largest one <= a.target whose units (rounded up per sequence)
// fit in a.target, i.e. one round of workgroups when the LDS cap allows it;
// ns/chunk receive this thread's sequences' plans.
template <int NT>
constexpr int plan_per_thread() { return kMaxBatch / NT; }

template <bool GATHER, int NT>
__device__ __forceinline__ void batch_plan(const AttnArgs& a, int* red, int (&ns)[plan_per_thread<NT>()],
                                           int (&chunk)[plan_per_thread<NT>()]) {
    constexpr int kPlanPerThread = plan_per_thread<NT>();
    int len[kPlanPerThread];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < kPlanPerThread; ++k) {
        const int b = k * NT + threadIdx.x;
        len[k] = b < a.batch ? seq_span<GATHER>(a, b).len : 0;
        mine += len[k];
    }
    const int total = wg_sum<NT>(mine, red);
    auto plan = [&](int t) {
        int u = 0;
#pragma unroll
        for (int k = 0; k < kPlanPerThread; ++k) {
            seq_plan(a, len[k], total, t, ns[k], chunk[k]);
            u += ns[k];
        }
        return wg_sum<NT>(u, red);
    };
    // (plan runs first also when every list is empty: it sets ns = 0 for all)
    if (plan(a.target) <= a.target || total <= 0) return;
    int lo = 1, hi = a.target - 1, best = 1;   // the unit count does not decrease with t
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        if (plan(mid) <= a.target) {
            best = mid;
            lo = mid + 1;
        } else {
            hi = mid - 1;
        }
    }
    plan(best);
}

// Rows of a 16-row tile a split partial keeps in the workspace: a single tile
// keeps only its M valid rows (e.g. the G rows of a drafting pass: a quarter
// of the bytes at G = 4), wider tiles all 16.  Partial slot layout, in float4
// units: ((d tile * MB + row tile) * 4 + lane / 16) * rows + lane % 16, for
// lane % 16 < rows; the (m, l) pairs: row tile * rows + lane % 16.
template <int MB>
__device__ __forceinline__ int part_rows(const AttnArgs& a) {
    return MB == 1 ? a.M : 16;
}

// Headroom of the lazily moved softmax reference (log2 units): block
// probabilities are at most 2^8, far inside bf16/fp32 range.
constexpr float kRescaleSlack = 8.f;

// Per-wave running state of the online softmax.
template <bool BF16, int D, int MB>
struct WaveState {
    Frag<BF16> qf[MB][D / 32];
    bool qvalid[MB];
    float cmask[MB];
    int rrow[MB];
    float m_run[MB], l_run[MB];
    f32x4_t o[D / 16][MB];
};

// PV step (fp32): acc += V^T(16 d x 16 pos) . P^T(16 pos x 16 rows).  Lane
// (lr, lg) supplies d (resp. row) lr and the k slots = positions 4*lg ..
// 4*lg+3, which is where the S^T accumulator left its probabilities.
__device__ __forceinline__ f32x4_t mfma_pv(const uint32_t (&vt)[4], const float (&p)[4], f32x4_t acc) {
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vt[m]), p[m], acc, 0, 0, 0);
    return acc;
}

// One 16-position block: S^T, collection, mask, online softmax, O^T += V^T P^T.
template <class GEO, bool BF16, int D, int MB, bool GATHER, bool COLLECT>
__device__ __forceinline__ void compute_block(const AttnArgs& a, WaveState<BF16, D, MB>& ws, int p0, int L,
                                              int end, int start, int lane, const unsigned char* stage,
                                              float* score_s) {
    constexpr int DC = D / 32, DB = D / 16, EPC = GEO::EPC;
    const int lr = lane & 15, lg = lane >> 4;
    const unsigned char* kt = stage;
    const unsigned char* vtile = stage + GEO::TILE;

    // S^T tile: 16 positions (MFMA rows) x 16 query rows per qb (MFMA columns).
    f32x4_t s[MB];
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) s[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < DC; ++ch) {
        Frag<BF16> kf;
        if constexpr (BF16) {
            const int cc = 4 * ch + lg;
            kf.u = *reinterpret_cast<const uint4*>(kt + lr * GEO::ROWB + ((cc ^ (lr & GEO::KSWZ)) << 4));
        } else {
            const int cc = 8 * ch + 2 * lg;
            kf.u[0] = *reinterpret_cast<const uint4*>(kt + lr * GEO::ROWB + ((cc ^ (lr & GEO::KSWZ)) << 4));
            kf.u[1] = *reinterpret_cast<const uint4*>(kt + lr * GEO::ROWB + (((cc + 1) ^ (lr & GEO::KSWZ)) << 4));
        }
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) s[qb] = mfma16(kf, ws.qf[qb][ch], s[qb]);
    }

    // Collect-2-Query: per prefix position, the collected rows' logits summed
    // over the query heads of this KV head (a reduction over the 16 lanes
    // holding the query rows), times s.
    if constexpr (COLLECT) {
        if (p0 < L) {
            float x[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                x[v] = 0.f;
#pragma unroll
                for (int qb = 0; qb < MB; ++qb) x[v] += ws.cmask[qb] * s[qb][v];
            }
            const float sum = row16_sum4(x, lr);      // position 4*lg + lr/4 of the block
            if ((lr & 3) == 0) {
                score_s[p0 - start + 4 * lg + (lr >> 2)] = a.scale * sum;
            }
        }
    }

    // Causal tail, end of the split, and (local mask) keys older than a row's band.
    const bool need_mask = GATHER ? (p0 + kAttnBlock > end)
                                  : (p0 + kAttnBlock > min(end, L + 1) || (a.window > 0 && p0 < L + a.W - a.window));
    if (need_mask) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int pos = p0 + 4 * lg + v;
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                const int last = L + ws.rrow[qb];
                const bool vis = pos < end && (GATHER || (pos <= last && (a.window <= 0 || pos > last - a.window)));
                if (!vis) s[qb][v] = kNegInf;
            }
        }
    }

    float pr[MB][4];
    bool rescale = false;
    float alpha[MB];
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        float mx = fmaxf(fmaxf(s[qb][0], s[qb][1]), fmaxf(s[qb][2], s[qb][3]));
        mx = pair32_max(pair16_max(mx));
        mx *= a.scale_log2;
        // Lazy rescaling: the running reference m moves (and O, l are
        // rescaled) only when a block's max exceeds it by more than
        // kRescaleSlack (log2 units), so the probabilities stay below
        // 2^kRescaleSlack and the O rescale runs a handful of times per
        // split instead of whenever any row's max creeps up.  The result is
        // the same softmax in real arithmetic ((m, l, O) stay consistent).
        const float m_old = ws.m_run[qb];
        const bool grow = mx > m_old + kRescaleSlack;     // also the first finite block
        const float m_new = grow ? mx : m_old;
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        alpha[qb] = grow ? fast_exp2(m_old - m_use) : 1.f;
        rescale |= grow;
        ws.m_run[qb] = m_new;
        float ls = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float p = fast_exp2(fmaf(s[qb][v], a.scale_log2, -m_use));
            pr[qb][v] = p;
            ls += p;
        }
        ws.l_run[qb] = fmaf(ws.l_run[qb], alpha[qb], ls);
    }
    if (__any(rescale)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) ws.o[db][qb] *= alpha[qb];
    }

    // O^T += V^T P^T over the 16 positions of the block.
    if constexpr (BF16) {
        // The V^T operand by transposed LDS reads (gfx950 ds_read_b64_tr_b16;
        // its lane mapping was checked on the device with a probe).  Within the
        // 16-lane group lg, lane (m, q) = (lr / 4, lr % 4) points at the four d
        // values 16*db + 4q .. +3 of position 4*lg + m; the read then hands
        // lane lr the values V[4*lg + e][16*db + lr], e = 0..3: its A-operand
        // k slots, the positions where the S^T accumulator left its P values.
        typedef short s16x4_t __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
        s16x4_t pb[MB];
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) {
            bf16x4_t t;
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = static_cast<__bf16>(pr[qb][i]);
            pb[qb] = __builtin_bit_cast(s16x4_t, t);
        }
        const int q = lr & 3;
        const unsigned char* vrow = vtile + (4 * lg + (lr >> 2)) * GEO::ROWB + 8 * (q & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const unsigned char* src = vrow + (((2 * db + (q >> 1)) ^ (GEO::SWZU * lg)) << 4);
            const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(src));
            const s16x4_t va = __builtin_bit_cast(s16x4_t, v);
#pragma unroll
            for (int qb = 0; qb < MB; ++qb)
                ws.o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[qb], ws.o[db][qb], 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + lr;
            const unsigned char* base = vtile + (4 * lg) * GEO::ROWB +
                                        (((d / EPC) ^ (GEO::SWZU * lg)) << 4) + (d % EPC) * GEO::ES;
            uint32_t vt[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) vt[m] = *reinterpret_cast<const uint32_t*>(base + m * GEO::ROWB);
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) ws.o[db][qb] = mfma_pv(vt, pr[qb], ws.o[db][qb]);
        }
    }
    lds_fence();   // this stage's reads are done before it is refilled
}

// One unit of the split kernel: positions [start, end) of sequence b (span
// sp; under a local mask no row sees a key before row 0's band, sp.lo) for KV
// head g and all query rows of the KV head.  The unit's partial goes to slot
// `slot` of (b, g).  Called by whole workgroups (every branch on its
// arguments is uniform); the LDS arrays are the kernel's.
template <bool BF16, int D, int MB, bool GATHER, bool COLLECT, bool PAIR>
__device__ __forceinline__ void split_unit(const AttnArgs& a, int g0, int b, int slot, int start, int end,
                                           const SeqSpan& sp, unsigned char* smem, int* idx_s, int* page_s,
                                           float* score_s) {
    constexpr int NT = kAttnWaves * 64;           // threads
    using GEO = Geo<BF16, D, MB, GATHER>;
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int DC = GEO::DC, DB = GEO::DB, NREG = GEO::NREG, NST = GEO::NST;
    constexpr int OPS = GEO::BLOCK_OPS;           // copies one wave issues per block
    // PAIR (gather only): waves 2i and 2i+1 take KV heads g0 and g0+1 of the
    // same rows, so a block's copies read 512 contiguous bytes of every row;
    // each head has two position groups.
    static_assert(!PAIR || GATHER, "head pairs are a gather layout");
    constexpr int NPG = PAIR ? kAttnWaves / 2 : kAttnWaves;    // position groups per KV head
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave
    const int pw = PAIR ? wv >> 1 : wv;                                  // its position group
    const int g = PAIR ? g0 + (wv & 1) : g0;                             // its KV head
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int seq0 = sp.seq0, n_b = sp.n_b, L = sp.L, ib0 = sp.ib0;
    if (n_b <= 0 || start >= end) return;                         // uniform per workgroup


    WaveState<BF16, D, MB> ws;
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        // B operand of S^T: query row 16*qb + lane%16, elements 32*ch + 8*(lane/16) .. +7
        const int j = 16 * qb + lr;
        const bool valid = j < a.M;
        const int r = valid ? j / a.G : a.W - 1;
        const int hl = valid ? j % a.G : 0;
        ws.rrow[qb] = r;
        ws.cmask[qb] = (COLLECT && valid && ((a.collect_mask >> r) & 1u)) ? 1.f : 0.f;
        // Padding rows load a real row (no divergent branch, so all loads stay
        // in flight together) and are zeroed afterwards.
        const T* qp = static_cast<const T*>(a.q) +
                      ((size_t)(b * a.W + r) * a.hq + (size_t)g * a.G + hl) * D + 8 * lg;
#pragma unroll
        for (int ch = 0; ch < DC; ++ch) ws.qf[qb][ch] = load_frag<BF16>(qp + 32 * ch);
        ws.qvalid[qb] = valid;
        ws.m_run[qb] = kNegInf;
        ws.l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) ws.o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // Gather mode: stage this split's index list (clamped into the sequence)
    // while the Q loads are in flight.
    const bool paged = a.page_shift >= 0;
    const int pmask = paged ? (1 << a.page_shift) - 1 : 0;
    int page0 = 0;
    if constexpr (GATHER) {
        constexpr int IPT = kMaxGatherChunk / NT;   // indices per thread
        int t[IPT];
#pragma unroll
        for (int e = 0; e < IPT; ++e) {   // clamped, branch-free: all loads in flight together
            const int i = min(e * NT + (int)threadIdx.x, end - start - 1);
            t[e] = min(max(a.indices[ib0 + start + i], 0), n_b - 1);
        }
        if (paged) {                      // position -> row of the page pool
            int pg[IPT];
#pragma unroll
            for (int e = 0; e < IPT; ++e)
                pg[e] = a.block_table[(size_t)b * a.max_pages + min(t[e] >> a.page_shift, a.max_pages - 1)];
#pragma unroll
            for (int e = 0; e < IPT; ++e)
                t[e] = (min(max(pg[e], 0), a.num_pages - 1) << a.page_shift) | (t[e] & pmask);
        }
#pragma unroll
        for (int e = 0; e < IPT; ++e) {
            const int i = e * NT + threadIdx.x;
            if (i < end - start) idx_s[i] = t[e];
        }
        __syncthreads();
    } else {
        if (paged) {                      // the pool pages of positions start .. end-1
            page0 = start >> a.page_shift;
            const int npg = min(((end - 1) >> a.page_shift) - page0 + 1, a.page_cap);
            for (int i = threadIdx.x; i < npg; i += blockDim.x) {
                const int pg = a.block_table[(size_t)b * a.max_pages + min(page0 + i, a.max_pages - 1)];
                page_s[i] = min(max(pg, 0), a.num_pages - 1);
            }
            __syncthreads();
        }
    }

    SplitCtx c;
    c.row_stride = a.hkv * D * GEO::ES;
    c.head_off = g * D * GEO::ES;
    const size_t first = paged ? 0 : (size_t)seq0 * c.row_stride;
    c.kbase = static_cast<const unsigned char*>(a.k) + first;
    c.vbase = static_cast<const unsigned char*>(a.v) + first;
    c.idx_s = idx_s;
    c.page_s = page_s;
    c.page0 = page0;
    c.page_shift = GATHER ? -1 : a.page_shift;
    c.start = start;
    c.end = end;

    // This position group's blocks are pw, pw+NPG, ...; a ring of NST
    // stages keeps NST-1 of them in flight.  No copy goes past the group's last
    // block, so the wait at the top of iteration jj counts the copies of the
    // blocks after jj that were issued: those of block jj+1 with a three-stage
    // ring unless jj is the last block, none otherwise.
    static_assert(NST == 2 || NST == 3, "the waits below count one or two stages");
    const int nblk = (end - start + kAttnBlock - 1) / kAttnBlock;
    const int nmine = pw < nblk ? (nblk - pw + NPG - 1) / NPG : 0;
    unsigned char* ring = smem + wv * (NST * GEO::STAGE);
    auto block_pos = [&](int jj) { return start + (pw + NPG * min(jj, nmine - 1)) * kAttnBlock; };
    auto issue = [&](int jj, unsigned char* stage) { issue_block<GEO, GATHER>(c, block_pos(jj), lane, stage); };
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
        if (st < nmine) issue(st, ring + st * GEO::STAGE);
    // Retire the Q loads here, where the compiler can see it (its wait also
    // covers the first blocks' copies, issued after them), so that its own
    // wait for them is not placed inside the block loop.
#pragma unroll
    for (int qb = 0; qb < MB; ++qb)
#pragma unroll
        for (int ch = 0; ch < DC; ++ch) {
            keep_live(ws.qf[qb][ch]);
            if (!ws.qvalid[qb]) ws.qf[qb][ch] = zero_frag<BF16>();
        }
    for (int jj = 0; jj < nmine; ++jj) {
        // this wave's copies of block jj have landed
        if (NST == 3 && jj + 1 < nmine) wait_vmem<(NST - 2) * OPS>();
        else wait_vmem<0>();
        if (jj + NST - 1 < nmine) issue(jj + NST - 1, ring + ((jj + NST - 1) % NST) * GEO::STAGE);
        compute_block<GEO, BF16, D, MB, GATHER, COLLECT>(a, ws, block_pos(jj), L, end, start, lane,
                                                         ring + (jj % NST) * GEO::STAGE, score_s);
    }
    wait_vmem<0>();
#ifdef VEGAS_PHASE_TRACE
    if (threadIdx.x == 0 && blockIdx.x < kTraceMax) g_trace_loop[blockIdx.x] = wall_clock64();
#endif

    // Row sums: each lane summed its own positions.
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        ws.l_run[qb] = pair32_sum(pair16_sum(ws.l_run[qb]));
    }

    // Tree merge of each KV head's position groups' (m, l, O) through LDS, in
    // fragment order (with head pairs, both heads' merges side by side).
    __syncthreads();
    float* fs = reinterpret_cast<float*>(smem);
    constexpr int SLOTF = GEO::MSLOT / 4;
    constexpr int HW = PAIR ? 2 : 1;              // heads per workgroup
    const int hsel = PAIR ? (wv & 1) : 0;
#pragma unroll
    for (int half = NPG / 2; half >= 1; half >>= 1) {
        if (pw >= half && pw < 2 * half) {
            float* slot = fs + ((pw - half) * HW + hsel) * SLOTF;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qb = 0; qb < MB; ++qb)
                    *reinterpret_cast<f32x4_t*>(slot + ((db * MB + qb) * 64 + lane) * 4) = ws.o[db][qb];
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                slot[NREG * 256 + qb * 64 + lane] = ws.m_run[qb];
                slot[NREG * 256 + (MB + qb) * 64 + lane] = ws.l_run[qb];
            }
        }
        __syncthreads();
        if (pw < half) {
            const float* slot = fs + (pw * HW + hsel) * SLOTF;
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                const float mb = slot[NREG * 256 + qb * 64 + lane];
                const float lb = slot[NREG * 256 + (MB + qb) * 64 + lane];
                const float mm = fmaxf(ws.m_run[qb], mb);
                if (mm != kNegInf) {
                    const float ca = fast_exp2(ws.m_run[qb] - mm);
                    const float cb = fast_exp2(mb - mm);
                    ws.m_run[qb] = mm;
                    ws.l_run[qb] = ca * ws.l_run[qb] + cb * lb;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const f32x4_t ob =
                            *reinterpret_cast<const f32x4_t*>(slot + ((db * MB + qb) * 64 + lane) * 4);
                        ws.o[db][qb] = ca * ws.o[db][qb] + cb * ob;
                    }
                }
            }
        }
        __syncthreads();
    }

    const int prow = part_rows<MB>(a);
    if (pw == 0 && lr < prow) {   // partials in the combine's layout: all MB row tiles of the workgroup
        const size_t slot_i = ((size_t)b * a.hkv + g) * a.nsplit + slot;
        f32x4_t* po = reinterpret_cast<f32x4_t*>(a.part_o) + slot_i * (DB * MB * 4 * prow);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) po[((db * MB + qb) * 4 + lg) * prow + lr] = ws.o[db][qb];
        if (lg == 0) {
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                float2* pml = reinterpret_cast<float2*>(a.part_ml) + slot_i * (MB * prow) + qb * prow + lr;
                *pml = make_float2(ws.m_run[qb], ws.l_run[qb]);
            }
        }
    }
    if (COLLECT && a.collect_mask != 0u) {
        // The split's collected scores (prefix positions only), written last:
        // a workgroup barrier waits for the workgroup's outstanding stores, and
        // none follows here.  16-byte stores from the first 16-byte boundary of
        // the destination on; score_s was complete at the merge's second barrier.
        float* dst = a.scores + (size_t)g * a.total_kv + seq0 + start;
        const int nsc = min(end, L) - start;
        const int peel = min((int)((4u - (uint32_t)(((uintptr_t)dst >> 2) & 3u)) & 3u), max(nsc, 0));
        if ((int)threadIdx.x < peel) dst[threadIdx.x] = score_s[threadIdx.x];
        const int nv = max(nsc - peel, 0) >> 2;
        float4* dv = reinterpret_cast<float4*>(dst + peel);
        for (int i = threadIdx.x; i < nv; i += blockDim.x) {
            const float* sp = score_s + peel + 4 * i;
            dv[i] = make_float4(sp[0], sp[1], sp[2], sp[3]);
        }
        for (int i = peel + 4 * nv + threadIdx.x; i < nsc; i += blockDim.x) dst[i] = score_s[i];
    }
}

template <bool BF16, int D, int MB, bool GATHER, bool COLLECT, bool PAIR>
__global__ void __launch_bounds__(kAttnWaves * 64)
attn_split_kernel(const AttnArgs a) {
    constexpr int NT = kAttnWaves * 64;           // threads
    constexpr int NWV = NT / 64;                  // waves
    using GEO = Geo<BF16, D, MB, GATHER>;
    constexpr int MERGE = (kAttnWaves / 2) * GEO::MSLOT;
    constexpr int MAIN = GEO::RING > MERGE ? GEO::RING : MERGE;

    __shared__ __attribute__((aligned(16))) unsigned char smem[MAIN];
    __shared__ int idx_s[GATHER ? kMaxGatherChunk : 1];
    // LDS sized at launch: the collected scores of the longest unit of the
    // plan (a.score_cap floats; collection only), written to HBM once a unit
    // is done, then a paged verification's page list (a host-planned 128K
    // verification takes 64 KB for its scores where a fixed buffer held 80).
    extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
    float* score_s = reinterpret_cast<float*>(dyn_lds);
    int* page_s = reinterpret_cast<int*>(dyn_lds + (COLLECT ? attn_score_lds_bytes(a.score_cap) : 0));

#ifdef VEGAS_PHASE_TRACE
    const unsigned long long trace_t0 = wall_clock64();
#endif
    // Fused selection: clear its histograms and counts (read after this launch).
    if (a.sel_zero)
        for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < a.sel_zero_n; i += gridDim.x * blockDim.x)
            a.sel_zero[i] = 0u;

    // Workgroup -> (KV head g, or heads g and g+1 with PAIR; its units).
    // Without a unit table a workgroup runs one unit (sequence b, split): the
    // units of all sequences' split plans, in order; workgroups past the last
    // unit have no work.  With the device plan, workgroup 0 publishes every
    // sequence's split count for the combine.
    __shared__ int plan_red[NWV];
    __shared__ int plan_s[3];
    const int hgroups = PAIR ? a.hkv / 2 : a.hkv;
#ifdef VEGAS_PHASE_TRACE
    const int hg = g_trace_rotate ? (blockIdx.x + blockIdx.x / hgroups) % hgroups : blockIdx.x % hgroups;
#else
    const int hg = blockIdx.x % hgroups;
#endif
    const int g = PAIR ? 2 * hg : hg;
    const int unit_id = blockIdx.x / hgroups;
    // This workgroup's units: entries k0 .. k0+nunits-1 of the unit table, or
    // the one unit (b, split) of the per-sequence plan.  One call site of
    // split_unit, so the kernel holds one copy of it.
    int k0 = 0, nunits = 1;
    int b = 0, split = 0, chunk = 0;
    SeqSpan sp{};
    if (a.hp.nwg > 0) {
        k0 = a.hp.wg_first[unit_id];
        nunits = a.hp.wg_first[unit_id + 1] - k0;
    } else if (a.hp.n > 0) {
        // Host plan: the unit's sequence, split and span are in the arguments.
        b = -1;
        for (int t = 0; t < a.hp.n; ++t)
            if (unit_id >= a.hp.first[t] && unit_id < a.hp.first[t + 1]) b = t;
        if (b < 0) return;                                        // uniform per workgroup
        split = unit_id - a.hp.first[b];
        chunk = a.hp.chunk[b];
        sp.seq0 = a.hp.seq0[b];
        sp.n_b = a.hp.n_b[b];
        sp.L = a.hp.L[b];
        sp.lo = a.hp.lo[b];
        sp.len = a.hp.len[b];
        sp.ib0 = a.hp.ib0[b];
    } else {
        constexpr int kPlanPerThread = plan_per_thread<NT>();
        int pns[kPlanPerThread], pch[kPlanPerThread];
        batch_plan<GATHER, NT>(a, plan_red, pns, pch);
        if (threadIdx.x == 0) plan_s[0] = -1;
        int before = 0;                                  // units of the sequences of earlier passes
#pragma unroll
        for (int k = 0; k < kPlanPerThread; ++k) {
            if (k * NT >= a.batch) break;                // uniform
            const int bb = k * NT + threadIdx.x;
            const int ns = pns[k];
            if (blockIdx.x == 0 && bb < a.batch) a.seq_splits[bb] = ns;
            int v = ns;                                  // inclusive scan of ns over the threads
            const int ln = threadIdx.x & 63;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(v, off);
                if (ln >= off) v += y;
            }
            __syncthreads();
            if (ln == 63) plan_red[threadIdx.x >> 6] = v;
            __syncthreads();
            int wbefore = 0, all = 0;
#pragma unroll
            for (int w = 0; w < NWV; ++w) {
                wbefore += (w < (int)(threadIdx.x >> 6)) ? plan_red[w] : 0;
                all += plan_red[w];
            }
            const int first_unit = before + wbefore + v - ns;
            if (ns > 0 && unit_id >= first_unit && unit_id < first_unit + ns) {
                plan_s[0] = bb;
                plan_s[1] = unit_id - first_unit;
                plan_s[2] = pch[k];
            }
            before += all;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(plan_s[0]);           // uniform: kept in scalar registers
        if (b < 0) return;                                        // uniform per workgroup
        split = __builtin_amdgcn_readfirstlane(plan_s[1]);
        chunk = __builtin_amdgcn_readfirstlane(plan_s[2]);
        sp = seq_span<GATHER>(a, b);
    }
    for (int i = 0; i < nunits; ++i) {
        int slot = split, start = sp.lo + split * chunk, end = min(start + chunk, sp.lo + sp.len);
        if (a.hp.nwg > 0) {
            const int k = k0 + i;
            b = a.hp.u_bs[k] & 31;
            slot = a.hp.u_bs[k] >> 5;
            start = a.hp.u_start[k];
            end = a.hp.u_end[k];
            sp.seq0 = a.hp.seq0[b];
            sp.n_b = a.hp.n_b[b];
            sp.L = a.hp.L[b];
            sp.lo = a.hp.lo[b];
            sp.len = a.hp.len[b];
            sp.ib0 = a.hp.ib0[b];
            if (i > 0) __syncthreads();                           // the previous unit's LDS reads are done
        }
        split_unit<BF16, D, MB, GATHER, COLLECT, PAIR>(a, g, b, slot, start, end, sp, smem, idx_s, page_s,
                                                       score_s);
    }
#ifdef VEGAS_PHASE_TRACE
    if (threadIdx.x == 0 && blockIdx.x < kTraceMax) {
        unsigned long long* r = g_trace[blockIdx.x];
        r[0] = trace_t0;
        r[1] = g_trace_loop[blockIdx.x];
        r[2] = wall_clock64();
        r[3] = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_ID: CU, SH, SE ids
        r[4] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
        r[5] = (unsigned long long)b;
        r[6] = (unsigned long long)split;
        r[7] = (unsigned long long)g;
    }
#endif
}

// Merge the split partials of one (sequence, KV head, 16-row tile, 16-wide d
// tile) and write the normalised output in the storage dtype.  Each lane of
// a wave owns one float4 of the fragment layout; the four waves take the
// splits in turn (four loads in flight each) and their partial merges are
// combined through LDS in a fixed order.
constexpr int kCombineWaves = 4;
static_assert(kCombineWaves == kAttnWaves, "batch_plan's workgroup reductions assume both kernels' width");

// KEYS (fused verification + selection): afterwards the workgroups run the
// selection's first step (sel_keys_chunk) over the (sequence, chunk) units
// of sa, the scores being complete once the split kernel has ended.
template <bool BF16, int D, int MB, bool GATHER, bool KEYS>
__global__ void __launch_bounds__(kCombineWaves * 64) attn_combine_kernel(const AttnArgs a, const SelectArgs sa) {
    constexpr int DB = D / 16;
    constexpr int NREG = DB * MB;
    constexpr int U = 4;
    __shared__ f32x4_t acc_s[kCombineWaves - 1][64];
    __shared__ float2 md_s[kCombineWaves - 1][64];
    __shared__ uint32_t keys_h[KEYS ? kSelBins : 1];
    static_assert(!KEYS || kCombineWaves * 64 == kSelThreads, "sel_keys_chunk takes kSelThreads threads");
    int wg = blockIdx.x;
    const int db = wg % DB;
    wg /= DB;
    const int qb = wg % MB;
    wg /= MB;
    const int g = wg % a.hkv;
    const int b = wg / a.hkv;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int j = 16 * qb + lr;

    // published by the split kernel, or known from the host plan
    const int nsv = a.hp.n > 0 ? a.hp.first[b + 1] - a.hp.first[b] : min(max(a.seq_splits[b], 0), a.nsplit);

    float mr = kNegInf, den = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const size_t slot0 = ((size_t)b * a.hkv + g) * a.nsplit;
    const float2* pml = reinterpret_cast<const float2*>(a.part_ml);
    const f32x4_t* po = reinterpret_cast<const f32x4_t*>(a.part_o);
    const int prow = part_rows<MB>(a);      // lanes of rows past it hold no partial (and no output)
    const bool kept = lr < prow;
    for (int s0 = wave; s0 < nsv; s0 += U * kCombineWaves) {
        float2 ml[U];
        f32x4_t ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = min(s0 + u * kCombineWaves, nsv - 1);
            ml[u] = kept ? pml[(slot0 + s) * (MB * prow) + qb * prow + lr] : make_float2(kNegInf, 0.f);
            ov[u] = kept ? po[(slot0 + s) * (NREG * 4 * prow) + ((db * MB + qb) * 4 + lg) * prow + lr]
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u * kCombineWaves >= nsv || ml[u].x == kNegInf) continue;
            if (ml[u].x > mr) {
                const float cf = fast_exp2(mr - ml[u].x);
                acc *= cf;
                den *= cf;
                mr = ml[u].x;
            }
            const float w = fast_exp2(ml[u].x - mr);
            acc += w * ov[u];
            den += w * ml[u].y;
        }
    }
    if (wave > 0) {
        acc_s[wave - 1][lane] = acc;
        md_s[wave - 1][lane] = make_float2(mr, den);
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kCombineWaves - 1; ++w) {
            const float2 md = md_s[w][lane];
            if (md.x == kNegInf) continue;
            const f32x4_t ob = acc_s[w][lane];
            const float mm = fmaxf(mr, md.x);
            const float ca = fast_exp2(mr - mm);
            const float cb = fast_exp2(md.x - mm);
            acc = ca * acc + cb * ob;
            den = ca * den + cb * md.y;
            mr = mm;
        }
        if (j < a.M) {
            const float inv = den > 0.f ? 1.f / den : 0.f;
            acc *= inv;
            const int r = j / a.G;
            const int hl = j % a.G;
            const size_t orow = ((size_t)(b * a.W + r) * a.hq + (size_t)g * a.G + hl) * D + 16 * db + 4 * lg;
            if constexpr (BF16) {
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                bf16x4_t h;
                h[0] = static_cast<__bf16>(acc[0]);
                h[1] = static_cast<__bf16>(acc[1]);
                h[2] = static_cast<__bf16>(acc[2]);
                h[3] = static_cast<__bf16>(acc[3]);
                *reinterpret_cast<bf16x4_t*>(static_cast<uint16_t*>(a.out) + orow) = h;
            } else {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + orow) = acc;
            }
        }
    }
    if constexpr (KEYS) {
        const int units = sa.batch * sa.nchunks;
        for (int u = blockIdx.x; u < units; u += gridDim.x) sel_keys_chunk(sa, u / sa.nchunks, u % sa.nchunks, keys_h);
    }
}

template <bool BF16, int D, int MB, bool GATHER, bool COLLECT, bool PAIR>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream, const SelectArgs* sel) {
    // (a host plan knows the exact workgroup count; the device plan's grid is its bound)
    const int per_head = a.hp.nwg > 0 ? a.hp.nwg : (a.hp.n > 0 ? a.hp.first[a.hp.n] : a.max_units);
    const unsigned split_grid = (unsigned)((PAIR ? a.hkv / 2 : a.hkv) * per_head);
    const unsigned comb_grid = (unsigned)(a.batch * a.hkv * MB * (D / 16));
    const size_t dyn = (COLLECT ? attn_score_lds_bytes(a.score_cap) : 0) +
                       (!GATHER && a.page_shift >= 0 ? (size_t)a.page_cap * sizeof(int) : 0);
    if (split_grid > 0)
        hipLaunchKernelGGL((attn_split_kernel<BF16, D, MB, GATHER, COLLECT, PAIR>), dim3(split_grid),
                           dim3(kAttnWaves * 64), dyn, stream, a);
    if (comb_grid > 0) {
        if constexpr (COLLECT && !GATHER) {
            if (sel) {
                hipLaunchKernelGGL((attn_combine_kernel<BF16, D, MB, GATHER, true>), dim3(comb_grid),
                                   dim3(kCombineWaves * 64), 0, stream, a, *sel);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((attn_combine_kernel<BF16, D, MB, GATHER, false>), dim3(comb_grid),
                           dim3(kCombineWaves * 64), 0, stream, a, SelectArgs{});
    }
    return hipGetLastError();
}

template <bool BF16, int D, bool GATHER, bool COLLECT>
hipError_t launch_mb(const AttnArgs& a, int mb, hipStream_t s, const SelectArgs* sel) {
    if constexpr (GATHER) {
        // head pairs for the one-tile drafting passes (G <= 16) at an even KV head count
        if (a.pair) {
            if (mb == 1 && a.hkv % 2 == 0) return launch_t<BF16, D, 1, true, false, true>(a, s, sel);
            return hipErrorInvalidValue;
        }
    }
    if (mb == 1) return launch_t<BF16, D, 1, GATHER, COLLECT, false>(a, s, sel);
    if (mb == 2) return launch_t<BF16, D, 2, GATHER, COLLECT, false>(a, s, sel);
    // fp32 at D = 128 stops at 32 rows per KV head (LDS budget).  Three and
    // four row tiles keep one wave per position group with all the tiles in
    // its registers (at most 256 VGPRs + 198 AGPRs, bf16 at D = 128).
    if constexpr (BF16 || D == 64) {
        if (mb == 3) return launch_t<BF16, D, 3, GATHER, COLLECT, false>(a, s, sel);
        if (mb == 4) return launch_t<BF16, D, 4, GATHER, COLLECT, false>(a, s, sel);
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool GATHER, bool COLLECT>
hipError_t launch_d(const AttnArgs& a, int d, int mb, hipStream_t s, const SelectArgs* sel) {
    if (d == 64) return launch_mb<BF16, 64, GATHER, COLLECT>(a, mb, s, sel);
    if (d == 128) return launch_mb<BF16, 128, GATHER, COLLECT>(a, mb, s, sel);
    return hipErrorInvalidValue;
}

}  // namespace

#ifdef VEGAS_PHASE_TRACE
extern "C" int vegas_trace_read(void* host, size_t bytes) {
    if (bytes > sizeof(g_trace)) return -1;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int vegas_trace_set_rotation(int rotate) {
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_trace_rotate), &rotate, sizeof(int), 0, hipMemcpyHostToDevice);
}
#endif

hipError_t launch_attn(const AttnArgs& a, bool bf16, int head_dim, int mblocks, bool gather,
                       bool collect, hipStream_t stream, const SelectArgs* sel) {
    if (gather) {
        return bf16 ? launch_d<true, true, false>(a, head_dim, mblocks, stream, nullptr)
                    : launch_d<false, true, false>(a, head_dim, mblocks, stream, nullptr);
    }
    if (collect) {
        return bf16 ? launch_d<true, false, true>(a, head_dim, mblocks, stream, sel)
                    : launch_d<false, false, true>(a, head_dim, mblocks, stream, sel);
    }
    return bf16 ? launch_d<true, false, false>(a, head_dim, mblocks, stream, nullptr)
                : launch_d<false, false, false>(a, head_dim, mblocks, stream, nullptr);
}

}  // namespace vegas
