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
// split).  Its four waves take 32-position blocks in turn.  All W*G query rows
// that share KV head g (at most 64) are processed together, so every K/V byte
// is read from HBM exactly once for all rows.  Per block and wave:
//   S^T[pos, row] = K[pos, :] . Q[row, :]         16x16x32 bf16 MFMA, K from
//                                                  registers (direct loads)
//   online softmax over positions (exp2 domain)    rows are MFMA columns, so a
//                                                  row max is in-lane + 2 shuffles
//   O^T[d, row] += V^T[d, pos] . P^T[pos, row]     V staged in LDS (swizzled),
//                                                  read transposed
// The P^T operand is the S^T accumulator itself: the k order of the MFMA is a
// free permutation, so the four S^T values a lane owns for each of two 16-row
// position tiles are exactly its eight k slots, and V^T is read in that order.
// Partials (m, l, O) of the four waves are merged in LDS and one partial per
// workgroup goes to the workspace; attn_combine merges the splits.
#include "internal.h"

namespace vegas {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// Eight operand elements owned by one lane.
template <bool BF16> struct Frag;
template <> struct Frag<true> { uint4 u; };
template <> struct Frag<false> { float f[8]; };

template <bool BF16>
__device__ __forceinline__ Frag<BF16> zero_frag() {
    Frag<BF16> r;
    if constexpr (BF16) {
        r.u = make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) r.f[i] = 0.f;
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
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        r.f[0] = a.x; r.f[1] = a.y; r.f[2] = a.z; r.f[3] = a.w;
        r.f[4] = b.x; r.f[5] = b.y; r.f[6] = b.z; r.f[7] = b.w;
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
#pragma unroll
    for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[m], b.f[m], c, 0, 0, 0);
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
#pragma unroll
        for (int i = 0; i < 8; ++i) r.f[i] = p[i];
    }
    return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x124>(x);   // row_ror 4
    x += dpp<0x128>(x);   // row_ror 8
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Compiler barrier that also drains outstanding LDS operations of this wave.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <bool BF16, int D, int MB>
struct Geo {
    static constexpr int ES = BF16 ? 2 : 4;       // element bytes
    static constexpr int DC = D / 32;             // k chunks of the QK^T contraction
    static constexpr int DB = D / 16;             // 16-wide d tiles of the PV product
    static constexpr int ROWB = D * ES;           // bytes of one K/V row of one head
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static constexpr int EPC = 16 / ES;           // elements per chunk
    static constexpr int RPI = 64 / CPR;          // V rows covered by one wave-wide 16-B load
    static constexpr int VLD = kAttnBlock / RPI;  // V loads per lane per block
    static constexpr int SWZU = 16 / EPC;         // chunks per 16-element d tile
    static constexpr int VBUF = kAttnBlock * ROWB;
    static constexpr int NREG = DB * MB;          // O^T fragments per lane
    static constexpr int MSLOT = (NREG * 4 + 2 * MB) * 64 * 4;
    static constexpr int MAIN = (kAttnWaves * VBUF > (kAttnWaves / 2) * MSLOT)
                                    ? kAttnWaves * VBUF
                                    : (kAttnWaves / 2) * MSLOT;
};

// Byte offset of chunk cc of V row `row` inside a wave's tile.  The chunk
// index is XOR-swizzled with the row's 4-row group so that the transposed
// reads of the PV operand (four lane groups reading rows 4 apart, same d)
// hit distinct LDS banks.
template <class GEO>
__device__ __forceinline__ int vtile_offset(int row, int cc) {
    return row * GEO::ROWB + ((cc ^ (GEO::SWZU * ((row >> 2) & 3))) << 4);
}

template <bool BF16, int D, int MB, bool GATHER, bool COLLECT>
__global__ void __launch_bounds__(kAttnWaves * 64)
attn_split_kernel(const AttnArgs a) {
    using GEO = Geo<BF16, D, MB>;
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    constexpr int DC = GEO::DC, DB = GEO::DB, CPR = GEO::CPR, EPC = GEO::EPC;
    constexpr int RPI = GEO::RPI, VLD = GEO::VLD, NREG = GEO::NREG;

    __shared__ __attribute__((aligned(16))) unsigned char smem[GEO::MAIN];
    __shared__ int idx_s[GATHER ? kMaxGatherChunk : 1];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15;
    const int lg = lane >> 4;

    int wg = blockIdx.x;
    const int g = wg % a.hkv;
    wg /= a.hkv;
    const int split = wg % a.nsplit;
    const int b = wg / a.nsplit;

    const int seq0 = a.cu_seqlens_k[b];
    const int n_b = a.cu_seqlens_k[b + 1] - seq0;
    int count, L, ib0 = 0;
    if constexpr (GATHER) {
        ib0 = a.cu_idx[b];
        count = a.cu_idx[b + 1] - ib0;
        L = 0;
    } else {
        count = n_b;
        L = n_b - a.W;
    }
    const int start = split * a.chunk;
    if (n_b <= 0 || start >= count) return;          // uniform per workgroup
    const int end = min(start + a.chunk, count);

    if constexpr (GATHER) {
        for (int i = threadIdx.x; i < end - start; i += blockDim.x) {
            const int t = a.indices[ib0 + start + i];
            idx_s[i] = min(max(t, 0), n_b - 1);
        }
        __syncthreads();
    }

    const T* __restrict__ kbase = static_cast<const T*>(a.k);
    const T* __restrict__ vbase = static_cast<const T*>(a.v);
    const int last_tok = a.total_kv - 1;
    auto token = [&](int p) -> int {
        const int pc = min(p, end - 1);
        int t;
        if constexpr (GATHER) t = seq0 + idx_s[pc - start];
        else t = seq0 + pc;
        return min(max(t, 0), last_tok);
    };

    // Q fragments (B operand of S^T): lane holds query row 16*qb + lr.
    Frag<BF16> qf[MB][DC];
    float cmask[MB];
    int rrow[MB];
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        const int j = 16 * qb + lr;
        const bool valid = j < a.M;
        const int r = valid ? j / a.G : a.W - 1;
        const int hl = valid ? j % a.G : 0;
        rrow[qb] = r;
        cmask[qb] = (COLLECT && valid && ((a.collect_mask >> r) & 1u)) ? 1.f : 0.f;
        const T* qp = static_cast<const T*>(a.q) +
                      ((size_t)(b * a.W + r) * a.hq + (size_t)g * a.G + hl) * D + 8 * lg;
#pragma unroll
        for (int c = 0; c < DC; ++c) qf[qb][c] = valid ? load_frag<BF16>(qp + 32 * c) : zero_frag<BF16>();
    }

    float m_run[MB], l_run[MB];
    f32x4_t o[DB][MB];
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        m_run[qb] = kNegInf;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    unsigned char* vtile = smem + wave * GEO::VBUF;
    const int nblk = (end - start + kAttnBlock - 1) / kAttnBlock;

    Frag<BF16> kc[2][DC];
    uint4 vc[VLD];
    auto load_block = [&](int p0, Frag<BF16> (&kf)[2][DC], uint4 (&vr)[VLD]) {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int tok = token(p0 + 16 * pb + lr);
            const T* kp = kbase + ((size_t)tok * a.hkv + g) * D + 8 * lg;
#pragma unroll
            for (int c = 0; c < DC; ++c) kf[pb][c] = load_frag<BF16>(kp + 32 * c);
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int row = lane / CPR + i * RPI;
            const int tok = token(p0 + row);
            vr[i] = *reinterpret_cast<const uint4*>(vbase + ((size_t)tok * a.hkv + g) * D +
                                                     (lane % CPR) * EPC);
        }
    };

    int bi = wave;
    if (bi < nblk) load_block(start + bi * kAttnBlock, kc, vc);
    for (; bi < nblk; bi += kAttnWaves) {
        const int p0 = start + bi * kAttnBlock;
        const bool more = bi + kAttnWaves < nblk;
        Frag<BF16> kn[2][DC];
        uint4 vn[VLD];
        if (more) load_block(p0 + kAttnWaves * kAttnBlock, kn, vn);

        // Stage this block's V tile in the wave's LDS buffer.
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int row = lane / CPR + i * RPI;
            *reinterpret_cast<uint4*>(vtile + vtile_offset<GEO>(row, lane % CPR)) = vc[i];
        }

        // S^T tile: positions (MFMA rows) x query rows (MFMA columns), raw dot products.
        f32x4_t s[2][MB];
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < DC; ++c) acc = mfma16(kc[pb][c], qf[qb][c], acc);
                s[pb][qb] = acc;
            }

        // Collect-2-Query: per prefix position, sum the logits of the collected
        // rows over the query heads of this KV head (a row reduction across the
        // 16 lanes that hold the query rows), scaled by s.
        if constexpr (COLLECT) {
            if (p0 < L) {
                float red[2][4];
#pragma unroll
                for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float x = 0.f;
#pragma unroll
                        for (int qb = 0; qb < MB; ++qb) x += cmask[qb] * s[pb][qb][v];
                        red[pb][v] = row16_sum(x);
                    }
                if (lr < 8) {
                    const int pb = lr >> 2, v = lr & 3;
                    float val = red[0][0];
                    val = (lr == 1) ? red[0][1] : val;
                    val = (lr == 2) ? red[0][2] : val;
                    val = (lr == 3) ? red[0][3] : val;
                    val = (lr == 4) ? red[1][0] : val;
                    val = (lr == 5) ? red[1][1] : val;
                    val = (lr == 6) ? red[1][2] : val;
                    val = (lr == 7) ? red[1][3] : val;
                    const int pos = p0 + 16 * pb + 4 * lg + v;
                    if (pos < L && pos < end) a.scores[(size_t)g * a.total_kv + seq0 + pos] = a.scale * val;
                }
            }
        }

        // Mask positions past the range and, for verification, past L + r.
        const bool need_mask = GATHER ? (p0 + kAttnBlock > end) : (p0 + kAttnBlock > min(end, L + 1));
        if (need_mask) {
#pragma unroll
            for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int pos = p0 + 16 * pb + 4 * lg + v;
#pragma unroll
                    for (int qb = 0; qb < MB; ++qb) {
                        const bool vis = pos < end && (GATHER || pos <= L + rrow[qb]);
                        if (!vis) s[pb][qb][v] = kNegInf;
                    }
                }
        }

        // Online softmax in the exp2 domain.
        float pr[MB][8];
        bool rescale = false;
        float alpha[MB];
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) {
            float mx = kNegInf;
#pragma unroll
            for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[pb][qb][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mx *= a.scale_log2;
            const float m_new = fmaxf(m_run[qb], mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            alpha[qb] = fast_exp2(m_run[qb] - m_use);
            rescale |= (alpha[qb] != 1.f);
            m_run[qb] = m_new;
            float ls = 0.f;
#pragma unroll
            for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float p = fast_exp2(fmaf(s[pb][qb][v], a.scale_log2, -m_use));
                    pr[qb][4 * pb + v] = p;
                    ls += p;
                }
            l_run[qb] = fmaf(l_run[qb], alpha[qb], ls);
        }
        if (__any(rescale)) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qb = 0; qb < MB; ++qb) o[db][qb] *= alpha[qb];
        }

        // O^T += V^T P^T.  k slot m of lane group lg is position 4*lg+m (m<4)
        // or 16+4*lg+(m-4) (m>=4): the S^T layout.
        Frag<BF16> pf[MB];
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) pf[qb] = pack_probs<BF16>(pr[qb]);
        lds_fence();
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + lr;
            const unsigned char* base = vtile + (4 * lg) * GEO::ROWB +
                                        (((d / EPC) ^ (GEO::SWZU * lg)) << 4) + (d % EPC) * GEO::ES;
            Frag<BF16> vt;
            if constexpr (BF16) {
                uint32_t e[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int row = (m < 4) ? m : 12 + m;
                    e[m] = *reinterpret_cast<const uint16_t*>(base + row * GEO::ROWB);
                }
                vt.u = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                  e[6] | (e[7] << 16));
            } else {
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int row = (m < 4) ? m : 12 + m;
                    vt.f[m] = *reinterpret_cast<const float*>(base + row * GEO::ROWB);
                }
            }
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) o[db][qb] = mfma16(vt, pf[qb], o[db][qb]);
        }
        lds_fence();

        if (more) {
#pragma unroll
            for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                for (int c = 0; c < DC; ++c) kc[pb][c] = kn[pb][c];
#pragma unroll
            for (int i = 0; i < VLD; ++i) vc[i] = vn[i];
        }
    }

    // Row sums: each lane summed its own positions.
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
        l_run[qb] += __shfl_xor(l_run[qb], 16);
        l_run[qb] += __shfl_xor(l_run[qb], 32);
    }

    // Tree merge of the waves' (m, l, O) through LDS, in fragment order.
    __syncthreads();
    float* fs = reinterpret_cast<float*>(smem);
    constexpr int SLOTF = GEO::MSLOT / 4;
#pragma unroll
    for (int half = kAttnWaves / 2; half >= 1; half >>= 1) {
        if (wave >= half && wave < 2 * half) {
            float* slot = fs + (wave - half) * SLOTF;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int qb = 0; qb < MB; ++qb)
                    *reinterpret_cast<f32x4_t*>(slot + ((db * MB + qb) * 64 + lane) * 4) = o[db][qb];
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                slot[NREG * 256 + qb * 64 + lane] = m_run[qb];
                slot[NREG * 256 + (MB + qb) * 64 + lane] = l_run[qb];
            }
        }
        __syncthreads();
        if (wave < half) {
            const float* slot = fs + wave * SLOTF;
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                const float mb = slot[NREG * 256 + qb * 64 + lane];
                const float lb = slot[NREG * 256 + (MB + qb) * 64 + lane];
                const float mm = fmaxf(m_run[qb], mb);
                if (mm != kNegInf) {
                    const float ca = fast_exp2(m_run[qb] - mm);
                    const float cb = fast_exp2(mb - mm);
                    m_run[qb] = mm;
                    l_run[qb] = ca * l_run[qb] + cb * lb;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const f32x4_t ob =
                            *reinterpret_cast<const f32x4_t*>(slot + ((db * MB + qb) * 64 + lane) * 4);
                        o[db][qb] = ca * o[db][qb] + cb * ob;
                    }
                }
            }
        }
        __syncthreads();
    }

    if (wave == 0) {
        const size_t slot = ((size_t)b * a.hkv + g) * a.nsplit + split;
        f32x4_t* po = reinterpret_cast<f32x4_t*>(a.part_o) + slot * (NREG * 64);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) po[(db * MB + qb) * 64 + lane] = o[db][qb];
        if (lg == 0) {
#pragma unroll
            for (int qb = 0; qb < MB; ++qb) {
                float2* pml = reinterpret_cast<float2*>(a.part_ml) + slot * (MB * 16) + qb * 16 + lr;
                *pml = make_float2(m_run[qb], l_run[qb]);
            }
        }
    }
}

// Merge the split partials of one (sequence, KV head, 16-row tile) and write
// the normalised output rows in the storage dtype.
template <bool BF16, int D, int MB, bool GATHER>
__global__ void __launch_bounds__(64 * (D / 16))
attn_combine_kernel(const AttnArgs a) {
    constexpr int DB = D / 16;
    constexpr int NREG = DB * MB;
    int wg = blockIdx.x;
    const int qb = wg % MB;
    wg /= MB;
    const int g = wg % a.hkv;
    const int b = wg / a.hkv;
    const int db = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int j = 16 * qb + lr;
    if (j >= a.M) return;

    const int n_b = a.cu_seqlens_k[b + 1] - a.cu_seqlens_k[b];
    const int count = GATHER ? (a.cu_idx[b + 1] - a.cu_idx[b]) : n_b;
    int nsv = (n_b > 0 && count > 0) ? (count + a.chunk - 1) / a.chunk : 0;
    nsv = min(nsv, a.nsplit);

    float mr = kNegInf, den = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const size_t slot0 = ((size_t)b * a.hkv + g) * a.nsplit;
    for (int s = 0; s < nsv; ++s) {
        const size_t slot = slot0 + s;
        const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[slot * (MB * 16) + j];
        if (ml.x == kNegInf) continue;
        const f32x4_t ov =
            reinterpret_cast<const f32x4_t*>(a.part_o)[slot * (NREG * 64) + (db * MB + qb) * 64 + lane];
        if (ml.x > mr) {
            const float c = fast_exp2(mr - ml.x);
            acc *= c;
            den *= c;
            mr = ml.x;
        }
        const float w = fast_exp2(ml.x - mr);
        acc += w * ov;
        den += w * ml.y;
    }
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

template <bool BF16, int D, int MB, bool GATHER, bool COLLECT>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
    const unsigned split_grid = (unsigned)(a.batch * a.hkv * a.nsplit);
    const unsigned comb_grid = (unsigned)(a.batch * a.hkv * MB);
    if (split_grid > 0)
        hipLaunchKernelGGL((attn_split_kernel<BF16, D, MB, GATHER, COLLECT>), dim3(split_grid),
                           dim3(kAttnWaves * 64), 0, stream, a);
    if (comb_grid > 0)
        hipLaunchKernelGGL((attn_combine_kernel<BF16, D, MB, GATHER>), dim3(comb_grid),
                           dim3(64 * (D / 16)), 0, stream, a);
    return hipGetLastError();
}

template <bool BF16, int D, bool GATHER, bool COLLECT>
hipError_t launch_mb(const AttnArgs& a, int mb, hipStream_t s) {
    switch (mb) {
        case 1: return launch_t<BF16, D, 1, GATHER, COLLECT>(a, s);
        case 2: return launch_t<BF16, D, 2, GATHER, COLLECT>(a, s);
        case 3: return launch_t<BF16, D, 3, GATHER, COLLECT>(a, s);
        case 4: return launch_t<BF16, D, 4, GATHER, COLLECT>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, bool GATHER, bool COLLECT>
hipError_t launch_d(const AttnArgs& a, int d, int mb, hipStream_t s) {
    if (d == 64) return launch_mb<BF16, 64, GATHER, COLLECT>(a, mb, s);
    if (d == 128) return launch_mb<BF16, 128, GATHER, COLLECT>(a, mb, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, bool bf16, int head_dim, int mblocks, bool gather,
                       bool collect, hipStream_t stream) {
    if (gather) {
        return bf16 ? launch_d<true, true, false>(a, head_dim, mblocks, stream)
                    : launch_d<false, true, false>(a, head_dim, mblocks, stream);
    }
    if (collect) {
        return bf16 ? launch_d<true, false, true>(a, head_dim, mblocks, stream)
                    : launch_d<false, false, true>(a, head_dim, mblocks, stream);
    }
    return bf16 ? launch_d<true, false, false>(a, head_dim, mblocks, stream)
                : launch_d<false, false, false>(a, head_dim, mblocks, stream);
}

}  // namespace vegas
