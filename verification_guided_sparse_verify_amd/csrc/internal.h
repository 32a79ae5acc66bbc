// Internal interface between the host API (api.cpp) and the kernel launchers
// (attn.hip, select.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vegas {

// Record `message` as the calling thread's last error detail (what
// vegas_last_error_message returns); returns `status`.
int set_last_error(int status, const char* message);

// Waves per attention workgroup and positions per wave iteration.
constexpr int kAttnWaves = 4;
constexpr int kAttnBlock = 16;
// Depth of each wave's LDS ring of K/V blocks: enough stages that the blocks
// in flight (all but the one being computed) hold at least 8 KB per wave,
// 32 KB per CU, where streaming reads saturate; deeper rings measured slower.
// 2 stages (one 8 KB block in flight) except bf16 at D = 64 (4 KB blocks): 3.
// Gathered rows (drafting passes, bf16) take 3 stages at any D: scattered
// rows come back slower than streamed ones, and two blocks in flight per
// wave read the drafting bytes faster (measured).
__host__ __device__ constexpr int attn_stages(bool bf16, int head_dim, bool gather = false) {
    return (bf16 && (head_dim == 64 || gather)) ? 3 : 2;
}
// Longest position range one workgroup takes in gather mode: its index list
// is staged in LDS.
constexpr int kMaxGatherChunk = 2048;
// Paged KV cache: LDS words set aside for a verification split's page list on
// top of its collected-score buffer.  Splits over small pages trade score
// buffer for page list (paged_split_cap below).
constexpr int kMaxPagesPerSplit = 2048;
constexpr int kMaxPageSize = 256;
// Largest batch the attention passes take (their split plan keeps a few
// sequences per thread in registers).
constexpr int kMaxBatch = 1024;

// Bytes of one workgroup's K/V ring.
__host__ __device__ constexpr int attn_ring_bytes(bool bf16, int head_dim, bool gather = false) {
    return kAttnWaves * attn_stages(bf16, head_dim, gather) * 2 * kAttnBlock * head_dim * (bf16 ? 2 : 4);
}
// Longest position range one workgroup takes in verification: the collected
// scores of its range are buffered in LDS next to the ring (144 KB in all of
// the 160 KB, leaving room for the wave merge of the widest row tiles and a
// paged cache's page list); a multiple of kAttnWaves*kAttnBlock.
__host__ __device__ constexpr int collect_chunk_cap(bool bf16, int head_dim) {
    return (144 * 1024 - attn_ring_bytes(bf16, head_dim)) / 4 / 64 * 64;
}
// LDS bytes of a split workgroup's collected-score buffer for units of at most
// `positions` positions (the buffer is sized at launch).
__host__ __device__ constexpr int attn_score_lds_bytes(int positions) {
    return (positions * 4 + 15) / 16 * 16;
}
// Pool pages a paged verification split of at most `positions` positions
// stages in LDS: a range of n positions starting anywhere touches at most
// (n - 1) / page + 2 pages.
__host__ __device__ constexpr int paged_list_words(int positions, int page_size) {
    return (positions - 1) / page_size + 2;
}
// Longest paged verification split: the collected-score buffer and the page
// list share the LDS that a contiguous split's score buffer and
// kMaxPagesPerSplit words would take, so splits over small pages stay long
// (1-token pages at D = 128, bf16: 11200 positions instead of ~2K); a
// multiple of kAttnWaves*kAttnBlock, at most collect_chunk_cap.
__host__ __device__ constexpr int paged_split_cap(bool bf16, int head_dim, int page_size) {
    const int cap = collect_chunk_cap(bf16, head_dim);
    const int budget = attn_score_lds_bytes(cap) + kMaxPagesPerSplit * 4;
    int n = cap;
    while (n > kAttnWaves * kAttnBlock && attn_score_lds_bytes(n) + paged_list_words(n, page_size) * 4 > budget)
        n -= kAttnWaves * kAttnBlock;
    return n;
}

// Split plan computed on the host from host copies of the sequence offsets,
// passed in the kernel arguments (batches of at most kHostPlanMax sequences):
// the kernels then start without reading offsets or planning on the device.
// It is the plan the device computes from the same offsets (same splits, so
// the same output bits).
constexpr int kHostPlanMax = 16;
// Unit table of a balanced host plan (see HostPlan::nwg).
constexpr int kHostUnitsMax = 96;
constexpr int kHostWgMax = 64;
struct HostPlan {
    int32_t n;                          // sequences; 0: the kernels plan on the device
    int32_t first[kHostPlanMax + 1];    // first (sequence, split) unit of each sequence, per KV head
    int32_t chunk[kHostPlanMax];        // positions per split
    // the sequence's span, as the device derives it (clamped offsets)
    int32_t seq0[kHostPlanMax], n_b[kHostPlanMax], L[kHostPlanMax];
    int32_t lo[kHostPlanMax], len[kHostPlanMax], ib0[kHostPlanMax];
    // Balanced plan (nwg > 0): per KV head, nwg workgroups each take an equal
    // slice of the sequences' positions laid end to end, one unit per sequence
    // the slice touches.  Workgroup w runs units wg_first[w] .. wg_first[w+1]-1;
    // unit u covers positions [u_start[u], u_end[u]) of sequence u_bs[u] & 31
    // and writes partial slot u_bs[u] >> 5 of that sequence (slots numbered
    // in position order; first[] then counts each sequence's units).
    int32_t nwg;
    int32_t wg_first[kHostWgMax + 1];
    int32_t u_bs[kHostUnitsMax], u_start[kHostUnitsMax], u_end[kHostUnitsMax];
};

// Arguments of the split attention kernel and of its combine kernel.
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* cu_seqlens_k;   // [batch+1]
    const int32_t* indices;        // gather: per-sequence lists
    const int32_t* cu_idx;         // gather: [batch+1]
    float* part_o;                 // [batch*hkv*nsplit][MB*16*D] (fragment order)
    float* part_ml;                // [batch*hkv*nsplit][MB*16][2] (max in log2 units, sum)
    float* scores;                 // collect: [hkv, total_kv]
    void* out;                     // [batch*W, hq, D]
    int32_t batch, hq, hkv, G, W, M;   // M = W*G query rows per KV head
    int32_t total_kv;
    // Split plan, derived per sequence on the device (each sequence gets a share
    // of `target` splits per KV head proportional to its positions, none longer
    // than chunk_cap): nsplit bounds any sequence's splits (the partial slots per
    // (sequence, KV head)); max_units bounds the sum over sequences (the grid).
    int32_t target;
    int32_t chunk_cap;             // multiple of kAttnWaves*kAttnBlock
    int32_t nsplit;
    int32_t max_units;
    int32_t* seq_splits;           // workspace [batch]: splits of each sequence (split kernel -> combine)
    int32_t score_cap;             // longest unit of the plan (<= chunk_cap): the collected-score LDS buffer
    float scale;                   // softmax scale s
    float scale_log2;              // s * log2(e)
    uint32_t collect_mask;
    // Paged KV cache (page_shift >= 0): k, v are pools [num_pages, page size, hkv, D];
    // position t of sequence b is row t % page of pool page block_table[b*max_pages + t/page].
    const int32_t* block_table;
    int32_t max_pages;
    int32_t num_pages;
    int32_t page_shift;            // log2(page size); -1: contiguous varlen cache
    int32_t page_cap;              // LDS words of a verification split's page list (paged only)
    int32_t window;                // verification local mask: row r sees keys (L+r-window, L+r]; 0: none
    int32_t pair;                  // gather: each workgroup takes KV heads g and g+1 (two waves each)
    // Fused selection (verification with collection only): the split kernel
    // clears sel_zero[0 .. sel_zero_n) and the combine kernel runs the
    // selection's first step on the finished scores.  NULL: not fused.
    uint32_t* sel_zero;
    int32_t sel_zero_n;
    HostPlan hp;
};

// Speculative-sampling acceptance: two launches over kAcceptChunk-token chunks.
constexpr int kAcceptChunk = 4096;
struct AcceptArgs {
    const float* p;                // [batch, gamma+1, vocab]
    const float* q;                // [batch, gamma, vocab]
    const int32_t* draft;          // [batch, gamma]
    const float* u_accept;         // [batch, gamma]
    const float* u_sample;         // [batch]
    int32_t* n_accepted;           // [batch]
    int32_t* next_token;           // [batch]
    uint64_t* part;                // workspace [batch][nchunks][2]: residual and target mass sums
    int32_t* first_rej;            // workspace [batch]
    int32_t batch, gamma, nchunks;
    int64_t vocab;
};
hipError_t launch_spec_accept(const AcceptArgs& a, hipStream_t stream);

// Query-agnostic sink-plus-recent index lists.
hipError_t launch_streaming_indices(int batch, int W, int sinks, const int32_t* cu_seqlens_k, int32_t total_kv,
                                    const int32_t* cu_idx, int32_t total_idx, int32_t* indices,
                                    hipStream_t stream);

struct SelectArgs {
    const float* scores;           // [hkv, total_kv]
    const int32_t* cu_seqlens_k;   // [batch+1]
    const int32_t* cu_k;           // [batch+1]
    int32_t* indices;              // [cu_k[batch]]
    uint32_t* keys;                // [total_kv] order-preserving image of S
    uint32_t* cand_key;            // [total_kv] threshold-bin candidates, per sequence at its offset
    int32_t* cand_pos;             // [total_kv]
    uint32_t* zeroed;              // [batch*kSelBins + batch]: histograms, then candidate counts
    uint32_t* seq_info;            // [batch][4]: top digit d1, count above d1, theta key
    uint32_t* chunk_above;         // [batch][nchunks]: positions above the threshold bin
    uint32_t* chunk_off;           // [batch][nchunks]: first output slot of the chunk
    uint32_t* chunk_ties;          // [batch][nchunks]: keys equal to theta the chunk contributes
    int32_t batch, hkv, W, total_kv;
    int32_t nchunks;               // chunks per sequence
    // Host copies of each sequence's clamped geometry (hg_n sequences, at most
    // kHostPlanMax; 0: read from cu_seqlens_k and cu_k on the device).
    int32_t hg_n;
    int32_t hg_seq0[kHostPlanMax], hg_L[kHostPlanMax], hg_k[kHostPlanMax], hg_kout[kHostPlanMax];
};

constexpr int kSelDigitBits = 12;
constexpr int kSelBins = 1 << kSelDigitBits;
constexpr int kSelThreads = 256;
constexpr int kSelPer = 8;                        // positions per thread per chunk
constexpr int kSelChunk = kSelThreads * kSelPer;  // positions per chunk workgroup
constexpr int kSelChunkShift = 11;
constexpr int kSelMaxChunks = 4096;               // longest prefix: kSelMaxChunks * kSelChunk

// sel: non-NULL for the fused verification + selection path (collect only).
hipError_t launch_attn(const AttnArgs& a, bool bf16, int head_dim, int mblocks, bool gather,
                       bool collect, hipStream_t stream, const SelectArgs* sel = nullptr);

// Words of a.zeroed: per-sequence histograms, then candidate counts.
__host__ __device__ constexpr int select_zeroed_words(int batch) { return batch * kSelBins + batch; }

// All four selection launches (zero, keys, cand, write) ...
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
// ... or the last two, after a fused verification pass did zero and keys ...
hipError_t launch_select_tail(const SelectArgs& a, hipStream_t stream);
// ... or the last three, after a verification pass that only cleared the histograms.
hipError_t launch_select_from_keys(const SelectArgs& a, hipStream_t stream);

}  // namespace vegas
