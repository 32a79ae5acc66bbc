// Host side of the C ABI declared in include/vegas.h: argument validation,
// launch planning (split sizes), workspace layout and dispatch.  Nothing here
// synchronises with the device or allocates device memory.
#include "vegas.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

vegas_status_t fail(vegas_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

}  // namespace

namespace vegas {
int set_last_error(int status, const char* message) {
    g_last_error = message;
    return status;
}
}  // namespace vegas

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups the split kernel should expose: one round on the 256 CUs (the
// kernel holds one workgroup per CU).  Each further round costs a workgroup's
// start-up and drain on the critical path, about 10 us at 128K positions.
constexpr int kRoundWorkgroups = 256;
// Most rounds of verification workgroups a plan aims for (see plan_attn).
constexpr int kMaxRounds = 4;

struct AttnPlan {
    bool pair = false;   // gather: workgroups take two KV heads (the split kernel's PAIR layout)
    int mb = 0;          // 16-row query tiles per KV head
    int target = 0;      // splits per KV head for the whole batch, shared by length
    int cap = 0;         // longest split
    int nsplit = 0;      // most splits one (sequence, KV head) can get: partial slots
    int max_units = 0;   // most (sequence, split) units over the batch: the grid per KV head
    size_t part_o = 0;   // bytes
    size_t part_ml = 0;  // bytes
    size_t splits = 0;   // bytes: per-sequence split counts
    size_t total() const { return align_up(part_o) + align_up(part_ml) + align_up(splits); }
};

// max_n: the most positions one sequence's pass covers.  The kernels derive
// each sequence's splits from the device-side lengths (seq_plan in attn.hip);
// this sizes the grid and the partial slots for any lengths up to max_n.
AttnPlan plan_attn(bool bf16, int batch, int hkv, int M, int head_dim, int max_n, bool gather,
                   int page_size = 0, int64_t total = -1) {
    AttnPlan p;
    p.mb = (M + 15) / 16;
    const int unit = vegas::kAttnWaves * vegas::kAttnBlock;
    const int64_t n = max_n > 0 ? max_n : 1;
    // Both caps are multiples of `unit`.  Verification uses the same plan with
    // and without collection, so the two give bit-identical outputs.
    int cap = gather ? vegas::kMaxGatherChunk : vegas::collect_chunk_cap(bf16, head_dim);
    if (!gather && page_size > 0) {
        // a paged split stages its page list in LDS beside the score buffer
        const int page_cap = vegas::paged_split_cap(bf16, head_dim, page_size);
        if (page_cap < cap) cap = page_cap;
    }
    p.cap = cap;
    // A drafting pass with one query tile and an even KV head count runs its
    // workgroups on head pairs: both heads' 256-byte slices of every gathered
    // row in one workgroup, 512 contiguous bytes a row (a gather probe read
    // the drafting bytes ~5% faster so); twice the splits per head then keep
    // one round of workgroups.
    p.pair = gather && p.mb == 1 && hkv % 2 == 0;
    const int groups = p.pair ? hkv / 2 : hkv;
    // Splits per KV head: one round of workgroups, or whole rounds when the
    // cap forces more splits than one round holds (long sequences over small
    // pages): a round and a half of equal splits takes as long as two rounds
    // of half-length ones.  Only for batches the host can plan (the partial
    // slots grow with the target per sequence), up to four rounds.  `total`
    // (rows of the call's cache) counts at most batch * max_n positions, the
    // bound a workspace query takes, so a call never needs more workspace
    // than the query gave.
    const int base = std::max(1, kRoundWorkgroups / groups);
    int rounds = 1;
    if (!gather && batch <= vegas::kHostPlanMax) {
        const int64_t bound = (int64_t)batch * n;
        const int64_t tot = total >= 0 ? std::min<int64_t>(total, bound) : bound;
        const int64_t need = (tot + cap - 1) / cap;
        rounds = (int)std::min<int64_t>(kMaxRounds, std::max<int64_t>(1, (need + base - 1) / base));
    }
    p.target = base * rounds;
    // Bounds of the device plan (seq_plan / batch_plan in attn.hip): a sequence
    // gets at most max(target + 1, ceil(len / cap)) splits (the float share can
    // round one up), the batch at most max(target, ceil(total / cap)) + 2 * batch.
    p.nsplit = (int)std::max<int64_t>(p.target + 1, (n + cap - 1) / cap);
    p.max_units = (int)std::max<int64_t>(p.target, (batch * n + cap - 1) / cap) + 2 * batch;
    // a single 16-row tile keeps only its M valid rows in a partial (part_rows in attn.hip)
    const size_t rows = p.mb == 1 ? (size_t)M : (size_t)p.mb * 16;
    const size_t slots = (size_t)batch * hkv * p.nsplit;
    p.part_o = slots * rows * head_dim * sizeof(float);
    p.part_ml = slots * rows * 2 * sizeof(float);
    p.splits = (size_t)batch * sizeof(int32_t);
    return p;
}

// Balanced verification plan for ragged batches.  The per-sequence plan gives
// every split to one sequence, so a batch of unequal lengths leaves some
// workgroups with much more than an equal share (1.23x for 16 lengths drawn
// log-uniform from 4K to 128K).  Here plan.target workgroups per KV head
// each take an equal slice of the sequences' positions laid end to end, one
// unit per sequence the slice touches.  It replaces the per-sequence plan
// when its largest workgroup load, counting kUnitCost positions for each
// unit's fixed work (query loads, ring fill, merge, stores), is at least 3%
// smaller.  The merge then groups positions differently, so results differ
// from the per-sequence plan's in rounding only.
void balance_plan(const AttnPlan& plan, int batch, const int* len, const int* ns, int64_t total,
                  vegas::HostPlan* hp) {
    constexpr int unit = vegas::kAttnWaves * vegas::kAttnBlock;
    constexpr int64_t kUnitCost = 512;
    int64_t prop_max = 0;
    for (int b = 0; b < batch; ++b)
        for (int i = 0; i < ns[b]; ++i)
            prop_max = std::max<int64_t>(prop_max, std::min<int64_t>(hp->chunk[b], len[b] - (int64_t)i * hp->chunk[b]));
    int64_t C = (total + plan.target - 1) / plan.target;
    C = std::min<int64_t>((C + unit - 1) / unit * unit, plan.cap);
    const int64_t nwg = (total + C - 1) / C;
    if (nwg > vegas::kHostWgMax) return;
    int64_t cum[vegas::kHostPlanMax + 1];
    cum[0] = 0;
    for (int b = 0; b < batch; ++b) cum[b + 1] = cum[b] + len[b];
    int pieces[vegas::kHostPlanMax] = {};
    int nu = 0;
    int64_t worst = 0;
    vegas::HostPlan t = *hp;
    for (int64_t w = 0; w < nwg; ++w) {
        const int64_t lo = w * C, hi = std::min(total, lo + C);
        t.wg_first[w] = nu;
        int64_t load = 0;
        for (int b = 0; b < batch; ++b) {
            const int64_t s = std::max(lo, cum[b]), e = std::min(hi, cum[b + 1]);
            if (s >= e) continue;
            if (nu == vegas::kHostUnitsMax || pieces[b] >= plan.nsplit) return;
            t.u_bs[nu] = b | (pieces[b]++ << 5);
            t.u_start[nu] = (int)(hp->lo[b] + (s - cum[b]));
            t.u_end[nu] = (int)(hp->lo[b] + (e - cum[b]));
            ++nu;
            load += (e - s) + kUnitCost;
        }
        worst = std::max(worst, load);
    }
    if (worst * 100 >= (prop_max + kUnitCost) * 97) return;
    t.wg_first[nwg] = nu;
    t.nwg = (int)nwg;
    t.first[0] = 0;
    for (int b = 0; b < batch; ++b) t.first[b + 1] = t.first[b] + pieces[b];
    *hp = t;
}

// Host-side split plan: the same plan the kernels derive on the device
// (seq_span, seq_plan and batch_plan in attn.hip), evaluated on host copies of
// the offsets, for batches of at most kHostPlanMax sequences.  The caller
// guarantees the host arrays hold the device arrays' values; lengths are
// clamped exactly as on the device.
void host_plan(const AttnPlan& plan, int batch, int W, int window, int32_t total_kv, const int32_t* cu_host,
               const int32_t* cu_idx_host, bool gather, vegas::HostPlan* hp) {
    constexpr int unit = vegas::kAttnWaves * vegas::kAttnBlock;
    int len[vegas::kHostPlanMax];
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) {
        const int seq0 = std::min(std::max(cu_host[b], 0), total_kv);
        const int n_b = std::min(std::max(cu_host[b + 1], seq0), total_kv) - seq0;
        hp->seq0[b] = seq0;
        hp->n_b[b] = n_b;
        if (gather) {
            hp->ib0[b] = cu_idx_host[b];
            hp->L[b] = 0;
            hp->lo[b] = 0;
            hp->len[b] = n_b > 0 ? std::max(cu_idx_host[b + 1] - cu_idx_host[b], 0) : 0;
        } else {
            hp->ib0[b] = 0;
            hp->L[b] = n_b - W;
            hp->lo[b] = window > 0 ? std::max(0, hp->L[b] - window + 1) : 0;
            hp->len[b] = std::max(n_b - hp->lo[b], 0);
        }
        len[b] = hp->len[b];
        total += len[b];
    }
    int ns[vegas::kHostPlanMax];
    auto eval = [&](int t) {
        int units = 0;
        for (int b = 0; b < batch; ++b) {
            if (len[b] <= 0) {
                ns[b] = 0;
                hp->chunk[b] = unit;
                continue;
            }
            int want = (int)(((int64_t)len[b] * t + total - 1) / total);
            want = std::max(std::max(want, 1), (len[b] + plan.cap - 1) / plan.cap);
            int chunk = (len[b] + want - 1) / want;
            chunk = (chunk + unit - 1) / unit * unit;
            hp->chunk[b] = chunk;
            ns[b] = std::min((len[b] + chunk - 1) / chunk, plan.nsplit);
            units += ns[b];
        }
        return units;
    };
    if (!(eval(plan.target) <= plan.target || total <= 0)) {
        int lo = 1, hi = plan.target - 1, best = 1;   // the unit count does not decrease with t
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (eval(mid) <= plan.target) {
                best = mid;
                lo = mid + 1;
            } else {
                hi = mid - 1;
            }
        }
        eval(best);
    }
    hp->first[0] = 0;
    for (int b = 0; b < batch; ++b) hp->first[b + 1] = hp->first[b] + ns[b];
    hp->n = batch;
    hp->nwg = 0;
    if (!gather && total > 0) balance_plan(plan, batch, len, ns, total, hp);
}

// Longest unit (split or balanced slice) of a host plan, in positions,
// rounded up to whole 16-position blocks: a unit's last block records the
// collected scores of all its 16 positions, also those past the unit's end,
// and the buffer must hold them (past it lies a paged verification's page
// list).
int longest_unit(const vegas::HostPlan& hp) {
    int m = 0;
    if (hp.nwg > 0) {
        for (int u = 0; u < hp.wg_first[hp.nwg]; ++u) m = std::max(m, hp.u_end[u] - hp.u_start[u]);
    } else {
        for (int b = 0; b < hp.n; ++b)
            if (hp.first[b + 1] > hp.first[b]) m = std::max(m, std::min(hp.chunk[b], hp.len[b]));
    }
    return (m + vegas::kAttnBlock - 1) / vegas::kAttnBlock * vegas::kAttnBlock;
}

// Host offsets: non-decreasing, within [0, total] (total < 0: no bound).
vegas_status_t check_host_offsets(const int32_t* cu, int batch, int64_t total, const char* name) {
    if (!cu) return fail(VEGAS_ERR_INVALID_ARGUMENT, "host %s is NULL", name);
    if (cu[0] < 0) return fail(VEGAS_ERR_INVALID_ARGUMENT, "host %s[0] = %d < 0", name, cu[0]);
    for (int b = 0; b < batch; ++b)
        if (cu[b + 1] < cu[b])
            return fail(VEGAS_ERR_INVALID_ARGUMENT, "host %s decreases at %d (%d -> %d)", name, b, cu[b], cu[b + 1]);
    if (total >= 0 && cu[batch] > total)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "host %s[batch] = %d exceeds %lld", name, cu[batch],
                    (long long)total);
    return VEGAS_OK;
}

vegas_status_t check_shape(const vegas_attn_shape_t* s) {
    if (!s) return fail(VEGAS_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (s->dtype != VEGAS_DTYPE_F32 && s->dtype != VEGAS_DTYPE_BF16)
        return fail(VEGAS_ERR_UNSUPPORTED, "dtype %d is not VEGAS_DTYPE_F32 or VEGAS_DTYPE_BF16", s->dtype);
    if (s->batch < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", s->batch);
    if (s->batch > vegas::kMaxBatch)
        return fail(VEGAS_ERR_UNSUPPORTED, "batch %d exceeds %d", s->batch, vegas::kMaxBatch);
    if (s->num_q_heads < 1 || s->num_kv_heads < 1)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Hq=%d, Hkv=%d)",
                    s->num_q_heads, s->num_kv_heads);
    if (s->num_q_heads % s->num_kv_heads != 0)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    s->num_q_heads, s->num_kv_heads);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(VEGAS_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", s->head_dim);
    if (!(s->softmax_scale > 0.f) || !std::isfinite(s->softmax_scale))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
    return VEGAS_OK;
}

// Query rows per KV head one workgroup can hold: 64, or 32 for fp32 at D = 128.
int max_rows(const vegas_attn_shape_t* s) {
    return (s->dtype == VEGAS_DTYPE_F32 && s->head_dim == 128) ? 32 : 64;
}

vegas_status_t check_gamma(int32_t gamma, const vegas_attn_shape_t* s) {
    if (gamma < 0 || gamma > 31) return fail(VEGAS_ERR_INVALID_ARGUMENT, "gamma %d outside 0..31", gamma);
    const int G = s->num_q_heads / s->num_kv_heads;
    if ((gamma + 1) * G > max_rows(s))
        return fail(VEGAS_ERR_UNSUPPORTED, "(gamma+1)*(Hq/Hkv) = %d exceeds %d query rows per KV head",
                    (gamma + 1) * G, max_rows(s));
    return VEGAS_OK;
}

// Kernels address K/V with 32-bit byte offsets from a sequence's first row.
bool rows_fit_32bit(const vegas_attn_shape_t* s, int64_t rows) {
    const int64_t es = s->dtype == VEGAS_DTYPE_BF16 ? 2 : 4;
    return rows * s->num_kv_heads * s->head_dim * es < (int64_t(1) << 32);
}

// log2 of the page size of a paged cache descriptor, after validation; -1 for NULL.
vegas_status_t check_pages(const vegas_paged_kv_t* pages, int32_t batch, int32_t max_seqlen_k, int* shift) {
    *shift = -1;
    if (!pages) return VEGAS_OK;
    const int ps = pages->page_size;
    if (ps < 1 || ps > vegas::kMaxPageSize || (ps & (ps - 1)) != 0)
        return fail(VEGAS_ERR_UNSUPPORTED, "page_size %d is not a power of two in 1..%d", ps, vegas::kMaxPageSize);
    if (!pages->block_table) return fail(VEGAS_ERR_INVALID_ARGUMENT, "block_table is NULL");
    if (pages->num_pages < 1 || (int64_t)pages->num_pages * ps >= (int64_t(1) << 31))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "num_pages %d gives an empty or over-long page pool",
                    pages->num_pages);
    if ((int64_t)pages->max_pages_per_seq * ps < max_seqlen_k)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_pages_per_seq %d x page_size %d < max_seqlen_k %d",
                    pages->max_pages_per_seq, ps, max_seqlen_k);
    (void)batch;
    int sh = 0;
    while ((1 << sh) < ps) ++sh;
    *shift = sh;
    return VEGAS_OK;
}

vegas_status_t hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(VEGAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return VEGAS_OK;
}

struct SelectPlan {
    int nchunks = 0;
    size_t keys = 0, cand_key = 0, cand_pos = 0, zeroed = 0, seq_info = 0, chunk = 0;
    size_t total() const {
        return align_up(keys) + align_up(cand_key) + align_up(cand_pos) + align_up(zeroed) +
               align_up(seq_info) + 3 * align_up(chunk);
    }
};

SelectPlan plan_select(int batch, int max_seqlen_k, int total_kv) {
    SelectPlan p;
    p.nchunks = (max_seqlen_k + vegas::kSelChunk - 1) / vegas::kSelChunk;
    p.keys = (size_t)total_kv * sizeof(uint32_t);
    p.cand_key = (size_t)total_kv * sizeof(uint32_t);
    p.cand_pos = (size_t)total_kv * sizeof(int32_t);
    p.zeroed = ((size_t)batch * vegas::kSelBins + batch) * sizeof(uint32_t);
    p.seq_info = (size_t)batch * 4 * sizeof(uint32_t);
    p.chunk = (size_t)batch * p.nchunks * sizeof(uint32_t);
    return p;
}

}  // namespace

extern "C" {

int32_t vegas_abi_version(void) { return VEGAS_ABI_VERSION; }

const char* vegas_status_string(vegas_status_t s) {
    switch (s) {
        case VEGAS_OK: return "VEGAS_OK";
        case VEGAS_ERR_INVALID_ARGUMENT: return "VEGAS_ERR_INVALID_ARGUMENT";
        case VEGAS_ERR_UNSUPPORTED: return "VEGAS_ERR_UNSUPPORTED";
        case VEGAS_ERR_WORKSPACE_TOO_SMALL: return "VEGAS_ERR_WORKSPACE_TOO_SMALL";
        case VEGAS_ERR_HIP: return "VEGAS_ERR_HIP";
    }
    return "VEGAS_ERR_UNKNOWN";
}

const char* vegas_last_error_message(void) { return g_last_error.c_str(); }

vegas_status_t vegas_verify_paged_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                 int32_t max_seqlen_k, int32_t page_size, size_t* bytes) {
    vegas_status_t st = check_shape(shape);
    if (st != VEGAS_OK) return st;
    if ((st = check_gamma(gamma, shape)) != VEGAS_OK) return st;
    if (!bytes) return fail(VEGAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (max_seqlen_k < gamma + 1)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_seqlen_k %d < gamma+1", max_seqlen_k);
    if (page_size < 0 || page_size > vegas::kMaxPageSize || (page_size & (page_size - 1)) != 0)
        return fail(VEGAS_ERR_UNSUPPORTED, "page_size %d is not 0 or a power of two up to %d", page_size,
                    vegas::kMaxPageSize);
    const int G = shape->num_q_heads / shape->num_kv_heads;
    *bytes = plan_attn(shape->dtype == VEGAS_DTYPE_BF16, shape->batch, shape->num_kv_heads, (gamma + 1) * G,
                       shape->head_dim, max_seqlen_k, false, page_size).total();
    return VEGAS_OK;
}

vegas_status_t vegas_verify_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                           int32_t max_seqlen_k, size_t* bytes) {
    return vegas_verify_paged_workspace_size(shape, gamma, max_seqlen_k, 0, bytes);
}

}  // extern "C"

namespace {

// Positions of one sequence a verification split plan has to cover.
int verify_span(int32_t max_seqlen_k, int32_t gamma, int32_t window) {
    return window > 0 ? std::min<int64_t>(max_seqlen_k, (int64_t)window + gamma) : max_seqlen_k;
}

vegas_status_t verify_impl(const vegas_attn_shape_t* shape, int32_t gamma, const void* q, const void* k,
                           const void* v, const vegas_paged_kv_t* pages, const int32_t* cu_seqlens_k,
                           int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask, float* scores,
                           void* out, void* workspace, size_t workspace_bytes, void* stream, int32_t window = 0,
                           const vegas::SelectArgs* fused = nullptr, const int32_t* cu_host = nullptr,
                           bool launch = true, bool keys_in_combine = true) {
    vegas_status_t st = check_shape(shape);
    if (st != VEGAS_OK) return st;
    if ((st = check_gamma(gamma, shape)) != VEGAS_OK) return st;
    const int W = gamma + 1;
    if (!q || !k || !v || !cu_seqlens_k || !out)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "q, k, v, cu_seqlens_k and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
    if (W < 32 && (collect_mask >> W) != 0u)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "collect_mask 0x%x has bits at rows >= gamma+1 = %d",
                    collect_mask, W);
    if (collect_mask != 0u && !scores)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "scores is NULL but collect_mask is non-zero");
    if (max_seqlen_k < W)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_seqlen_k %d < gamma+1 = %d", max_seqlen_k, W);
    if (total_kv < shape->batch * W)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "total_kv %d < batch*(gamma+1)", total_kv);
    int shift = -1;
    if ((st = check_pages(pages, shape->batch, max_seqlen_k, &shift)) != VEGAS_OK) return st;
    if (!pages && !rows_fit_32bit(shape, max_seqlen_k))
        return fail(VEGAS_ERR_UNSUPPORTED, "one sequence's K/V rows span 4 GiB or more");
    const int G = shape->num_q_heads / shape->num_kv_heads;
    if (window < 0) return fail(VEGAS_ERR_INVALID_ARGUMENT, "window %d < 0", window);
    if (window > 0 && collect_mask != 0u)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "collection is not defined under a local mask");
    const AttnPlan plan = plan_attn(shape->dtype == VEGAS_DTYPE_BF16, shape->batch, shape->num_kv_heads, W * G,
                                    shape->head_dim, verify_span(max_seqlen_k, gamma, window), false,
                                    pages ? pages->page_size : 0, total_kv);
    if (workspace_bytes < plan.total())
        return fail(VEGAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.total(),
                    workspace_bytes);
    if (!workspace) return fail(VEGAS_ERR_INVALID_ARGUMENT, "workspace is NULL");

    vegas::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu_seqlens_k = cu_seqlens_k;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(plan.part_o));
    a.seq_splits = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(plan.part_o) +
                                              align_up(plan.part_ml));
    a.scores = scores;
    a.out = out;
    a.batch = shape->batch;
    a.hq = shape->num_q_heads;
    a.hkv = shape->num_kv_heads;
    a.G = G;
    a.W = W;
    a.M = W * G;
    a.total_kv = total_kv;
    a.target = plan.target;
    a.chunk_cap = plan.cap;
    a.nsplit = plan.nsplit;
    a.max_units = plan.max_units;
    a.scale = shape->softmax_scale;
    a.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
    a.collect_mask = collect_mask;
    a.window = window;
    a.page_shift = shift;
    if (pages) {
        a.block_table = pages->block_table;
        a.max_pages = pages->max_pages_per_seq;
        a.num_pages = pages->num_pages;
    }
    if (fused) {
        a.sel_zero = fused->zeroed;
        a.sel_zero_n = vegas::select_zeroed_words(fused->batch);
    }
    if (cu_host) {
        if ((st = check_host_offsets(cu_host, shape->batch, total_kv, "cu_seqlens_k")) != VEGAS_OK) return st;
        for (int b = 0; b < shape->batch; ++b) {
            const int len = cu_host[b + 1] - cu_host[b];
            if (len < W || len > max_seqlen_k)
                return fail(VEGAS_ERR_INVALID_ARGUMENT, "sequence %d has %d rows, outside [gamma+1, max_seqlen_k] = "
                            "[%d, %d]", b, len, W, max_seqlen_k);
        }
        if (shape->batch <= vegas::kHostPlanMax)
            host_plan(plan, shape->batch, W, window, total_kv, cu_host, nullptr, false, &a.hp);
    }
    a.score_cap = plan.cap;
    if (a.hp.n > 0) a.score_cap = longest_unit(a.hp);
    a.page_cap = pages ? vegas::paged_list_words(plan.cap, 1 << shift) : 0;
    if (!launch) return VEGAS_OK;                  // arguments checked only
    // (fused without the keys step: the split kernel still clears the selection's histograms)
    return hip_status(vegas::launch_attn(a, shape->dtype == VEGAS_DTYPE_BF16, shape->head_dim, plan.mb,
                                         false, collect_mask != 0u, static_cast<hipStream_t>(stream),
                                         keys_in_combine ? fused : nullptr),
                      "verify launch");
}

// Selection arguments over a workspace of at least plan.total() bytes.
vegas::SelectArgs select_args(const SelectPlan& plan, int32_t batch, int32_t num_kv_heads, int32_t gamma,
                              const float* scores, const int32_t* cu_seqlens_k, int32_t total_kv,
                              const int32_t* cu_k, int32_t* indices, void* workspace) {
    char* ws = static_cast<char*>(workspace);
    auto take = [&ws](size_t n) {
        char* p = ws;
        ws += align_up(n);
        return p;
    };
    vegas::SelectArgs a{};
    a.scores = scores;
    a.cu_seqlens_k = cu_seqlens_k;
    a.cu_k = cu_k;
    a.indices = indices;
    a.keys = reinterpret_cast<uint32_t*>(take(plan.keys));
    a.cand_key = reinterpret_cast<uint32_t*>(take(plan.cand_key));
    a.cand_pos = reinterpret_cast<int32_t*>(take(plan.cand_pos));
    a.zeroed = reinterpret_cast<uint32_t*>(take(plan.zeroed));
    a.seq_info = reinterpret_cast<uint32_t*>(take(plan.seq_info));
    a.chunk_above = reinterpret_cast<uint32_t*>(take(plan.chunk));
    a.chunk_off = reinterpret_cast<uint32_t*>(take(plan.chunk));
    a.chunk_ties = reinterpret_cast<uint32_t*>(take(plan.chunk));
    a.batch = batch;
    a.hkv = num_kv_heads;
    a.W = gamma + 1;
    a.total_kv = total_kv;
    a.nchunks = plan.nchunks;
    return a;
}

vegas_status_t decode_impl(const vegas_attn_shape_t* shape, const void* q, const void* k, const void* v,
                           const vegas_paged_kv_t* pages, const int32_t* cu_seqlens_k, int32_t total_kv,
                           const int32_t* indices, const int32_t* cu_idx, int32_t max_idx, void* out,
                           void* workspace, size_t workspace_bytes, void* stream,
                           const vegas_host_offsets_t* host = nullptr) {
    size_t need = 0;
    vegas_status_t st = vegas_sparse_decode_workspace_size(shape, max_idx, &need);
    if (st != VEGAS_OK) return st;
    if (!q || !k || !v || !cu_seqlens_k || !cu_idx || !out)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "q, k, v, cu_seqlens_k, cu_idx and out must be non-NULL");
    if (max_idx > 0 && !indices) return fail(VEGAS_ERR_INVALID_ARGUMENT, "indices is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
    if (total_kv < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "total_kv must be >= 1");
    int shift = -1;
    if ((st = check_pages(pages, shape->batch, 1, &shift)) != VEGAS_OK) return st;
    if (workspace_bytes < need)
        return fail(VEGAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!workspace) return fail(VEGAS_ERR_INVALID_ARGUMENT, "workspace is NULL");
    const int G = shape->num_q_heads / shape->num_kv_heads;
    const AttnPlan plan = plan_attn(shape->dtype == VEGAS_DTYPE_BF16, shape->batch, shape->num_kv_heads, G,
                                    shape->head_dim, max_idx, true);
    vegas::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu_seqlens_k = cu_seqlens_k;
    a.indices = indices;
    a.cu_idx = cu_idx;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(plan.part_o));
    a.seq_splits = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(plan.part_o) +
                                              align_up(plan.part_ml));
    a.scores = nullptr;
    a.out = out;
    a.batch = shape->batch;
    a.hq = shape->num_q_heads;
    a.hkv = shape->num_kv_heads;
    a.G = G;
    a.W = 1;
    a.M = G;
    a.total_kv = total_kv;
    a.target = plan.target;
    a.chunk_cap = plan.cap;
    a.nsplit = plan.nsplit;
    a.max_units = plan.max_units;
    a.scale = shape->softmax_scale;
    a.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
    a.collect_mask = 0u;
    a.page_shift = shift;
    a.pair = plan.pair ? 1 : 0;
    if (pages) {
        a.block_table = pages->block_table;
        a.max_pages = pages->max_pages_per_seq;
        a.num_pages = pages->num_pages;
    }
    if (host) {
        if ((st = check_host_offsets(host->cu_seqlens_k, shape->batch, total_kv, "cu_seqlens_k")) != VEGAS_OK ||
            (st = check_host_offsets(host->cu_idx, shape->batch, -1, "cu_idx")) != VEGAS_OK)
            return st;
        for (int b = 0; b < shape->batch; ++b)
            if (host->cu_idx[b + 1] - host->cu_idx[b] > max_idx)
                return fail(VEGAS_ERR_INVALID_ARGUMENT, "list %d holds %d indices, more than max_idx %d", b,
                            host->cu_idx[b + 1] - host->cu_idx[b], max_idx);
        if (shape->batch <= vegas::kHostPlanMax)
            host_plan(plan, shape->batch, 1, 0, total_kv, host->cu_seqlens_k, host->cu_idx, true, &a.hp);
    }
    return hip_status(vegas::launch_attn(a, shape->dtype == VEGAS_DTYPE_BF16, shape->head_dim, plan.mb,
                                         true, false, static_cast<hipStream_t>(stream)),
                      "sparse decode launch");
}

}  // namespace

extern "C" {

vegas_status_t vegas_verify_attn(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                 const void* k, const void* v, const int32_t* cu_seqlens_k,
                                 int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                 float* scores, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return verify_impl(shape, gamma, q, k, v, nullptr, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask,
                       scores, out, workspace, workspace_bytes, stream);
}

vegas_status_t vegas_verify_attn_paged(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                       const void* k, const void* v, const vegas_paged_kv_t* pages,
                                       const int32_t* cu_seqlens_k, int32_t max_seqlen_k, int32_t total_kv,
                                       uint32_t collect_mask, float* scores, void* out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (!pages) return fail(VEGAS_ERR_INVALID_ARGUMENT, "pages is NULL");
    return verify_impl(shape, gamma, q, k, v, pages, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask,
                       scores, out, workspace, workspace_bytes, stream);
}

vegas_status_t vegas_verify_local_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                 int32_t max_seqlen_k, int32_t window, size_t* bytes) {
    if (window < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "window %d < 1", window);
    if (max_seqlen_k < gamma + 1)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_seqlen_k %d < gamma+1", max_seqlen_k);
    return vegas_verify_workspace_size(shape, gamma, verify_span(max_seqlen_k, gamma, window), bytes);
}

vegas_status_t vegas_verify_attn_local(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                       const void* k, const void* v, const int32_t* cu_seqlens_k,
                                       int32_t max_seqlen_k, int32_t total_kv, int32_t window, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (window < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "window %d < 1", window);
    return verify_impl(shape, gamma, q, k, v, nullptr, cu_seqlens_k, max_seqlen_k, total_kv, 0u, nullptr, out,
                       workspace, workspace_bytes, stream, window);
}

vegas_status_t vegas_streaming_indices(int32_t batch, int32_t gamma, int32_t sinks, const int32_t* cu_seqlens_k,
                                       int32_t total_kv, const int32_t* cu_idx, int32_t total_idx,
                                       int32_t* indices, void* stream) {
    if (batch < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (gamma < 0 || gamma > 31) return fail(VEGAS_ERR_INVALID_ARGUMENT, "gamma %d outside 0..31", gamma);
    if (sinks < 0 || total_kv < 1 || total_idx < 0)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "sinks, total_idx must be >= 0 and total_kv >= 1");
    if (!cu_seqlens_k || !cu_idx || (total_idx > 0 && !indices))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "cu_seqlens_k, cu_idx and indices must be non-NULL");
    return hip_status(vegas::launch_streaming_indices(batch, gamma + 1, sinks, cu_seqlens_k, total_kv, cu_idx,
                                                      total_idx, indices, static_cast<hipStream_t>(stream)),
                      "streaming indices launch");
}

vegas_status_t vegas_spec_accept_workspace_size(int32_t batch, int32_t vocab, size_t* bytes) {
    if (batch < 1 || vocab < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "batch and vocab must be >= 1");
    if (!bytes) return fail(VEGAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
    const size_t nch = ((size_t)vocab + vegas::kAcceptChunk - 1) / vegas::kAcceptChunk;
    *bytes = align_up((size_t)batch * nch * 2 * sizeof(uint64_t)) + align_up((size_t)batch * sizeof(int32_t));
    return VEGAS_OK;
}

vegas_status_t vegas_spec_accept(int32_t batch, int32_t gamma, int32_t vocab, const float* p, const float* q,
                                 const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                                 int32_t* n_accepted, int32_t* next_token, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    size_t need = 0;
    vegas_status_t st = vegas_spec_accept_workspace_size(batch, vocab, &need);
    if (st != VEGAS_OK) return st;
    if (gamma < 0 || gamma > 31) return fail(VEGAS_ERR_INVALID_ARGUMENT, "gamma %d outside 0..31", gamma);
    if (!p || !u_sample || !n_accepted || !next_token || (gamma > 0 && (!q || !draft_tokens || !u_accept)))
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "p, q, draft_tokens, u_accept, u_sample, n_accepted and "
                                                "next_token must be non-NULL (q, draft_tokens, u_accept may be "
                                                "NULL when gamma is 0)");
    if (workspace_bytes < need)
        return fail(VEGAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!workspace) return fail(VEGAS_ERR_INVALID_ARGUMENT, "workspace is NULL");
    vegas::AcceptArgs a{};
    a.p = p;
    a.q = q;
    a.draft = draft_tokens;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.n_accepted = n_accepted;
    a.next_token = next_token;
    a.batch = batch;
    a.gamma = gamma;
    a.vocab = vocab;
    a.nchunks = (int)(((int64_t)vocab + vegas::kAcceptChunk - 1) / vegas::kAcceptChunk);
    a.part = static_cast<uint64_t*>(workspace);
    a.first_rej = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             align_up((size_t)batch * a.nchunks * 2 * sizeof(uint64_t)));
    return hip_status(vegas::launch_spec_accept(a, static_cast<hipStream_t>(stream)), "spec accept launch");
}

vegas_status_t vegas_select_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t gamma,
                                           int32_t max_seqlen_k, int32_t total_kv, size_t* bytes) {
    if (batch < 1 || num_kv_heads < 1) return fail(VEGAS_ERR_INVALID_ARGUMENT, "batch and num_kv_heads must be >= 1");
    if (gamma < 0 || gamma > 31) return fail(VEGAS_ERR_INVALID_ARGUMENT, "gamma %d outside 0..31", gamma);
    if (max_seqlen_k < gamma + 1 || total_kv < 1)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_seqlen_k must be >= gamma+1 and total_kv >= 1");
    if ((int64_t)max_seqlen_k > (int64_t)vegas::kSelMaxChunks * vegas::kSelChunk)
        return fail(VEGAS_ERR_UNSUPPORTED, "max_seqlen_k %d exceeds %d", max_seqlen_k,
                    vegas::kSelMaxChunks * vegas::kSelChunk);
    if (!bytes) return fail(VEGAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = plan_select(batch, max_seqlen_k, total_kv).total();
    return VEGAS_OK;
}

vegas_status_t vegas_select_topk(int32_t batch, int32_t num_kv_heads, int32_t gamma,
                                 const float* scores, const int32_t* cu_seqlens_k,
                                 int32_t max_seqlen_k, int32_t total_kv, const int32_t* cu_k,
                                 int32_t* indices, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    size_t need = 0;
    vegas_status_t st = vegas_select_workspace_size(batch, num_kv_heads, gamma, max_seqlen_k, total_kv, &need);
    if (st != VEGAS_OK) return st;
    if (!scores || !cu_seqlens_k || !cu_k || !indices)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "scores, cu_seqlens_k, cu_k and indices must be non-NULL");
    if (workspace_bytes < need)
        return fail(VEGAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!workspace) return fail(VEGAS_ERR_INVALID_ARGUMENT, "workspace is NULL");
    const vegas::SelectArgs a = select_args(plan_select(batch, max_seqlen_k, total_kv), batch, num_kv_heads,
                                            gamma, scores, cu_seqlens_k, total_kv, cu_k, indices, workspace);
    return hip_status(vegas::launch_select(a, static_cast<hipStream_t>(stream)), "select launch");
}

vegas_status_t vegas_verify_select_workspace_size(const vegas_attn_shape_t* shape, int32_t gamma,
                                                  int32_t max_seqlen_k, int32_t total_kv, size_t* bytes) {
    if (!bytes) return fail(VEGAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
    size_t vb = 0, sb = 0;
    vegas_status_t st = vegas_verify_workspace_size(shape, gamma, max_seqlen_k, &vb);
    if (st != VEGAS_OK) return st;
    st = vegas_select_workspace_size(shape->batch, shape->num_kv_heads, gamma, max_seqlen_k, total_kv, &sb);
    if (st != VEGAS_OK) return st;
    *bytes = align_up(vb) + sb;
    return VEGAS_OK;
}

}  // extern "C"

namespace {

// Which launches of the one-call verification + selection a call issues: all
// of them (the keys step in the verification combine kernel); the
// verification kernels only (the split kernel clearing the selection's
// histograms); or the selection's remaining steps (keys, candidates, write).
enum class Part { kAll, kBegin, kEnd };

vegas_status_t verify_select_impl(const vegas_attn_shape_t* shape, int32_t gamma, const void* q, const void* k,
                                  const void* v, const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                  int32_t total_kv, uint32_t collect_mask, const int32_t* cu_k, float* scores,
                                  int32_t* indices, void* out, void* workspace, size_t workspace_bytes,
                                  void* stream, const vegas_host_offsets_t* host, Part part = Part::kAll) {
    size_t need = 0, vb = 0;
    vegas_status_t st = vegas_verify_select_workspace_size(shape, gamma, max_seqlen_k, total_kv, &need);
    if (st != VEGAS_OK) return st;
    if (collect_mask == 0u)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "collect_mask is 0: there are no scores to select from");
    if (!cu_k || !indices) return fail(VEGAS_ERR_INVALID_ARGUMENT, "cu_k and indices must be non-NULL");
    if (workspace_bytes < need)
        return fail(VEGAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need, workspace_bytes);
    if (!workspace) return fail(VEGAS_ERR_INVALID_ARGUMENT, "workspace is NULL");
    vegas_verify_workspace_size(shape, gamma, max_seqlen_k, &vb);
    vegas::SelectArgs sa =
        select_args(plan_select(shape->batch, max_seqlen_k, total_kv), shape->batch, shape->num_kv_heads, gamma,
                    scores, cu_seqlens_k, total_kv, cu_k, indices, static_cast<char*>(workspace) + align_up(vb));
    if (host) {
        if ((st = check_host_offsets(host->cu_idx, shape->batch, -1, "cu_k")) != VEGAS_OK) return st;
        if (shape->batch <= vegas::kHostPlanMax && host->cu_seqlens_k) {
            // each sequence's clamped selection geometry, as seq_geo derives it on the device
            const int kend = std::max(host->cu_idx[shape->batch], 0);
            for (int b = 0; b < shape->batch; ++b) {
                const int seq0 = std::min(std::max(host->cu_seqlens_k[b], 0), total_kv);
                const int end = std::min(std::max(host->cu_seqlens_k[b + 1], seq0), total_kv);
                const int L = std::min(std::max(end - seq0 - (gamma + 1), 0), sa.nchunks * vegas::kSelChunk);
                const int kout = std::min(std::max(host->cu_idx[b], 0), kend);
                sa.hg_seq0[b] = seq0;
                sa.hg_L[b] = L;
                sa.hg_kout[b] = kout;
                sa.hg_k[b] = std::min(std::min(std::max(host->cu_idx[b + 1] - kout, 0), L), kend - kout);
            }
            sa.hg_n = shape->batch;
        }
    }
    if ((st = verify_impl(shape, gamma, q, k, v, nullptr, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask,
                          scores, out, workspace, vb, stream, 0, &sa, host ? host->cu_seqlens_k : nullptr,
                          part != Part::kEnd, part == Part::kAll)) != VEGAS_OK)
        return st;
    if (part == Part::kBegin) return VEGAS_OK;
    if (part == Part::kEnd)
        return hip_status(vegas::launch_select_from_keys(sa, static_cast<hipStream_t>(stream)), "select launch");
    return hip_status(vegas::launch_select_tail(sa, static_cast<hipStream_t>(stream)), "select launch");
}

}  // namespace

extern "C" {

vegas_status_t vegas_verify_select(const vegas_attn_shape_t* shape, int32_t gamma, const void* q, const void* k,
                                   const void* v, const int32_t* cu_seqlens_k, int32_t max_seqlen_k,
                                   int32_t total_kv, uint32_t collect_mask, const int32_t* cu_k, float* scores,
                                   int32_t* indices, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    return verify_select_impl(shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, cu_k,
                              scores, indices, out, workspace, workspace_bytes, stream, nullptr);
}

vegas_status_t vegas_verify_attn_hostplan(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                          const void* k, const void* v, const int32_t* cu_seqlens_k,
                                          int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                          float* scores, void* out, void* workspace, size_t workspace_bytes,
                                          void* stream, const vegas_host_offsets_t* host) {
    if (!host || !host->cu_seqlens_k) return fail(VEGAS_ERR_INVALID_ARGUMENT, "host cu_seqlens_k must be non-NULL");
    return verify_impl(shape, gamma, q, k, v, nullptr, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, scores,
                       out, workspace, workspace_bytes, stream, 0, nullptr, host->cu_seqlens_k);
}

vegas_status_t vegas_verify_hostplan_info(const vegas_attn_shape_t* shape, int32_t gamma, int32_t max_seqlen_k,
                                          int32_t total_kv, const vegas_host_offsets_t* host, int32_t* balanced,
                                          int32_t* workgroups) {
    vegas_status_t st = check_shape(shape);
    if (st != VEGAS_OK) return st;
    if ((st = check_gamma(gamma, shape)) != VEGAS_OK) return st;
    if (!balanced || !workgroups) return fail(VEGAS_ERR_INVALID_ARGUMENT, "balanced and workgroups must be non-NULL");
    if (!host || !host->cu_seqlens_k) return fail(VEGAS_ERR_INVALID_ARGUMENT, "host cu_seqlens_k must be non-NULL");
    const int W = gamma + 1;
    if (max_seqlen_k < W) return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_seqlen_k %d < gamma+1 = %d", max_seqlen_k, W);
    if ((st = check_host_offsets(host->cu_seqlens_k, shape->batch, total_kv, "cu_seqlens_k")) != VEGAS_OK) return st;
    for (int b = 0; b < shape->batch; ++b) {
        const int len = host->cu_seqlens_k[b + 1] - host->cu_seqlens_k[b];
        if (len < W || len > max_seqlen_k)
            return fail(VEGAS_ERR_INVALID_ARGUMENT, "sequence %d has %d rows, outside [gamma+1, max_seqlen_k] = [%d, %d]",
                        b, len, W, max_seqlen_k);
    }
    const int G = shape->num_q_heads / shape->num_kv_heads;
    const AttnPlan plan = plan_attn(shape->dtype == VEGAS_DTYPE_BF16, shape->batch, shape->num_kv_heads, W * G,
                                    shape->head_dim, max_seqlen_k, false, 0, total_kv);
    *balanced = 0;
    *workgroups = plan.max_units;
    if (shape->batch <= vegas::kHostPlanMax) {
        vegas::HostPlan hp{};
        host_plan(plan, shape->batch, W, 0, total_kv, host->cu_seqlens_k, nullptr, false, &hp);
        *balanced = hp.nwg > 0 ? 1 : 0;
        *workgroups = hp.nwg > 0 ? hp.nwg : hp.first[hp.n];
    }
    return VEGAS_OK;
}

vegas_status_t vegas_verify_select_hostplan(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                            const void* k, const void* v, const int32_t* cu_seqlens_k,
                                            int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                            const int32_t* cu_k, float* scores, int32_t* indices, void* out,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            const vegas_host_offsets_t* host) {
    if (!host || !host->cu_seqlens_k || !host->cu_idx)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "host offsets (cu_seqlens_k and cu_idx = cu_k) must be non-NULL");
    return verify_select_impl(shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, cu_k,
                              scores, indices, out, workspace, workspace_bytes, stream, host);
}

vegas_status_t vegas_verify_select_begin_hostplan(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                                  const void* k, const void* v, const int32_t* cu_seqlens_k,
                                                  int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                                  const int32_t* cu_k, float* scores, int32_t* indices, void* out,
                                                  void* workspace, size_t workspace_bytes, void* stream,
                                                  const vegas_host_offsets_t* host) {
    if (!host || !host->cu_seqlens_k || !host->cu_idx)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "host offsets (cu_seqlens_k and cu_idx = cu_k) must be non-NULL");
    return verify_select_impl(shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, cu_k,
                              scores, indices, out, workspace, workspace_bytes, stream, host, Part::kBegin);
}

vegas_status_t vegas_verify_select_end_hostplan(const vegas_attn_shape_t* shape, int32_t gamma, const void* q,
                                                const void* k, const void* v, const int32_t* cu_seqlens_k,
                                                int32_t max_seqlen_k, int32_t total_kv, uint32_t collect_mask,
                                                const int32_t* cu_k, float* scores, int32_t* indices, void* out,
                                                void* workspace, size_t workspace_bytes, void* stream,
                                                const vegas_host_offsets_t* host) {
    if (!host || !host->cu_seqlens_k || !host->cu_idx)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "host offsets (cu_seqlens_k and cu_idx = cu_k) must be non-NULL");
    return verify_select_impl(shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, cu_k,
                              scores, indices, out, workspace, workspace_bytes, stream, host, Part::kEnd);
}

vegas_status_t vegas_sparse_decode_workspace_size(const vegas_attn_shape_t* shape, int32_t max_idx,
                                                  size_t* bytes) {
    vegas_status_t st = check_shape(shape);
    if (st != VEGAS_OK) return st;
    if (!bytes) return fail(VEGAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (max_idx < 0) return fail(VEGAS_ERR_INVALID_ARGUMENT, "max_idx %d < 0", max_idx);
    const int G = shape->num_q_heads / shape->num_kv_heads;
    if (G > max_rows(shape))
        return fail(VEGAS_ERR_UNSUPPORTED, "Hq/Hkv = %d exceeds %d", G, max_rows(shape));
    *bytes = plan_attn(shape->dtype == VEGAS_DTYPE_BF16, shape->batch, shape->num_kv_heads, G, shape->head_dim,
                       max_idx, true).total();
    return VEGAS_OK;
}

vegas_status_t vegas_sparse_decode_attn(const vegas_attn_shape_t* shape, const void* q, const void* k,
                                        const void* v, const int32_t* cu_seqlens_k, int32_t total_kv,
                                        const int32_t* indices, const int32_t* cu_idx, int32_t max_idx,
                                        void* out, void* workspace, size_t workspace_bytes,
                                        void* stream) {
    return decode_impl(shape, q, k, v, nullptr, cu_seqlens_k, total_kv, indices, cu_idx, max_idx, out,
                       workspace, workspace_bytes, stream);
}

vegas_status_t vegas_sparse_decode_attn_hostplan(const vegas_attn_shape_t* shape, const void* q, const void* k,
                                                 const void* v, const int32_t* cu_seqlens_k, int32_t total_kv,
                                                 const int32_t* indices, const int32_t* cu_idx, int32_t max_idx,
                                                 void* out, void* workspace, size_t workspace_bytes, void* stream,
                                                 const vegas_host_offsets_t* host) {
    if (!host || !host->cu_seqlens_k || !host->cu_idx)
        return fail(VEGAS_ERR_INVALID_ARGUMENT, "host offsets (cu_seqlens_k and cu_idx) must be non-NULL");
    return decode_impl(shape, q, k, v, nullptr, cu_seqlens_k, total_kv, indices, cu_idx, max_idx, out,
                       workspace, workspace_bytes, stream, host);
}

vegas_status_t vegas_sparse_decode_attn_paged(const vegas_attn_shape_t* shape, const void* q, const void* k,
                                              const void* v, const vegas_paged_kv_t* pages,
                                              const int32_t* cu_seqlens_k, int32_t total_kv,
                                              const int32_t* indices, const int32_t* cu_idx, int32_t max_idx,
                                              void* out, void* workspace, size_t workspace_bytes,
                                              void* stream) {
    if (!pages) return fail(VEGAS_ERR_INVALID_ARGUMENT, "pages is NULL");
    return decode_impl(shape, q, k, v, pages, cu_seqlens_k, total_kv, indices, cu_idx, max_idx, out,
                       workspace, workspace_bytes, stream);
}

}  // extern "C"
