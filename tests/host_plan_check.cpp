// Host-side check of the launch planning in csrc/api.cpp, built for the CPU
// (with AddressSanitizer and UndefinedBehaviorSanitizer by the test that
// compiles it).  The kernel launchers are replaced by stubs that capture the
// arguments the host computed; nothing touches a GPU.
//
// For seeded random batches (1..1024 sequences, empty and short sequences,
// ragged and equal lengths, paged caches of 1..256-token pages, local
// windows, up to 64 query rows per KV head) every entry point that plans is
// called with valid arguments, and the captured plan is checked against the
// bounds the kernels rely on:
//   - the grid and the partial slots: no sequence needs more splits than
//     nsplit, the whole batch no more units than max_units (the device plan,
//     evaluated here in the same integer arithmetic), and the host plan's
//     units fit the grid it launches;
//   - coverage: the splits of every sequence cover its positions exactly,
//     none is empty and none is longer than the LDS buffers allow (the
//     collected-score buffer, in whole 16-position blocks, the staged index
//     list, the staged page list);
//   - the balanced plan's tables: workgroups, units and slot numbers within
//     their fixed arrays;
//   - the workspace: partials, split counts and the selection's buffers lie
//     inside the bytes the workspace query returned;
//   - the selection's per-sequence geometry: k within the prefix, outputs
//     within the packed list, chunks within the write kernel's LDS tables.
// Prints "ok <cases>" and exits 0, or prints the first violation and exits 1.
#include "api.cpp"

#include <cstdlib>
#include <random>
#include <vector>

namespace {

struct Captured {
    bool attn = false, sel_tail = false, sel_full = false;
    vegas::AttnArgs a{};
    bool bf16 = false, gather = false, collect = false, fused = false;
    int head_dim = 0, mb = 0;
    vegas::SelectArgs s{};
};
Captured g_cap;

}  // namespace

namespace vegas {
hipError_t launch_attn(const AttnArgs& a, bool bf16, int head_dim, int mblocks, bool gather, bool collect,
                       hipStream_t, const SelectArgs* sel) {
    g_cap.attn = true;
    g_cap.a = a;
    g_cap.bf16 = bf16;
    g_cap.head_dim = head_dim;
    g_cap.mb = mblocks;
    g_cap.gather = gather;
    g_cap.collect = collect;
    g_cap.fused = sel != nullptr;
    return hipSuccess;
}
hipError_t launch_select(const SelectArgs& a, hipStream_t) {
    g_cap.sel_full = true;
    g_cap.s = a;
    return hipSuccess;
}
hipError_t launch_select_tail(const SelectArgs& a, hipStream_t) {
    g_cap.sel_tail = true;
    g_cap.s = a;
    return hipSuccess;
}
hipError_t launch_select_from_keys(const SelectArgs& a, hipStream_t) {
    g_cap.sel_tail = true;
    g_cap.s = a;
    return hipSuccess;
}
hipError_t launch_spec_accept(const AcceptArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_streaming_indices(int, int, int, const int32_t*, int32_t, const int32_t*, int32_t, int32_t*,
                                    hipStream_t) {
    return hipSuccess;
}
}  // namespace vegas

// Only reached on a launch error, which the stubs never return.
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace {

long long g_cases = 0;
long long g_balanced = 0;   // balanced host plans checked
long long g_multiround = 0; // verification plans over more than one round of workgroups

[[noreturn]] void violation(const char* what, const std::string& detail) {
    std::printf("VIOLATION after %lld cases: %s\n%s\n", g_cases, what, detail.c_str());
    std::fflush(stdout);
    std::exit(1);
}

#define REQUIRE(cond, ...)                                                   \
    do {                                                                     \
        if (!(cond)) {                                                       \
            char buf_[512];                                                  \
            std::snprintf(buf_, sizeof buf_, __VA_ARGS__);                   \
            violation(#cond, ctx + " | " + buf_);                            \
        }                                                                    \
    } while (0)

std::mt19937_64 rng;
int64_t uni(int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); }
double unif() { return std::uniform_real_distribution<double>(0.0, 1.0)(rng); }

// The device's split plan (seq_plan and batch_plan in attn.hip) for any batch
// size, in the same integer arithmetic; ns_raw is a sequence's split count
// before the kernel's clamp to nsplit.
struct DevPlan {
    std::vector<int> ns_raw, chunk;
    long long units = 0;
};
DevPlan device_plan(const std::vector<int>& len, int target, int cap) {
    constexpr int unit = vegas::kAttnWaves * vegas::kAttnBlock;
    const int B = (int)len.size();
    long long total = 0;
    for (int x : len) total += x;
    DevPlan p;
    p.ns_raw.assign(B, 0);
    p.chunk.assign(B, unit);
    auto eval = [&](int t) {
        long long units = 0;
        for (int b = 0; b < B; ++b) {
            if (len[b] <= 0) {
                p.ns_raw[b] = 0;
                p.chunk[b] = unit;
                continue;
            }
            int want = (int)(((long long)len[b] * t + total - 1) / total);
            want = std::max(std::max(want, 1), (len[b] + cap - 1) / cap);
            int chunk = (len[b] + want - 1) / want;
            chunk = (chunk + unit - 1) / unit * unit;
            p.chunk[b] = chunk;
            p.ns_raw[b] = (len[b] + chunk - 1) / chunk;
            units += p.ns_raw[b];
        }
        return units;
    };
    // units are computed with the clamp to nsplit on the device; checking the
    // unclamped counts against nsplit below makes the clamp a no-op
    if (!(eval(target) <= target || total <= 0)) {
        int lo = 1, hi = target - 1, best = 1;
        while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (eval(mid) <= target) {
                best = mid;
                lo = mid + 1;
            } else {
                hi = mid - 1;
            }
        }
        eval(best);
    }
    p.units = 0;
    for (int x : p.ns_raw) p.units += x;
    return p;
}

struct Case {
    int dtype, B, hq, hkv, D, gamma, page, window;
    std::vector<int32_t> cu, cuk;
    int max_seqlen, total_kv, max_k;
    std::string ctx;
};

// Positions one sequence's pass covers, as seq_span derives them.
void spans(const Case& c, bool gather, std::vector<int>& len, std::vector<int>& lo) {
    len.assign(c.B, 0);
    lo.assign(c.B, 0);
    const int W = c.gamma + 1;
    for (int b = 0; b < c.B; ++b) {
        const int seq0 = std::min(std::max(c.cu[b], 0), c.total_kv);
        const int n_b = std::min(std::max(c.cu[b + 1], seq0), c.total_kv) - seq0;
        if (gather) {
            len[b] = n_b > 0 ? std::max(c.cuk[b + 1] - c.cuk[b], 0) : 0;
        } else {
            const int L = n_b - W;
            lo[b] = c.window > 0 ? std::max(0, L - c.window + 1) : 0;
            len[b] = std::max(n_b - lo[b], 0);
        }
    }
}

// Pages a split [start, end) of a paged verification stages in LDS.
int pages_spanned(int start, int end, int page) {
    return (end - 1) / page - start / page + 1;
}

void check_attn(const Case& c, bool gather, size_t ws_bytes, const char* entry, int page = 0) {
    const std::string ctx = c.ctx + " entry=" + entry;
    REQUIRE(g_cap.attn, "no attention launch");
    const vegas::AttnArgs& a = g_cap.a;
    const int B = c.B;
    const int G = c.hq / c.hkv;
    const int M = gather ? G : (c.gamma + 1) * G;
    const int mb = g_cap.mb;
    REQUIRE(mb * 16 >= M, "row tiles %d for %d rows", mb, M);
    REQUIRE(mb >= 1 && mb <= 4, "tile count %d", mb);
    const bool bf16 = c.dtype == VEGAS_DTYPE_BF16;
    const int cap = a.chunk_cap;
    const int lds_cap = gather ? vegas::kMaxGatherChunk : vegas::collect_chunk_cap(bf16, c.D);
    REQUIRE(cap > 0 && cap <= lds_cap && cap % (vegas::kAttnWaves * vegas::kAttnBlock) == 0, "cap %d (LDS %d)",
            cap, lds_cap);

    // workspace: partial slots, (m, l) pairs, split counts
    const size_t slots = (size_t)B * c.hkv * a.nsplit;
    const char* w0 = reinterpret_cast<const char*>(a.part_o);
    const char* wml = reinterpret_cast<const char*>(a.part_ml);
    const char* wsp = reinterpret_cast<const char*>(a.seq_splits);
    // a single row tile keeps its M valid rows, wider tiles all 16 rows of each tile
    const size_t rows = mb == 1 ? (size_t)M : (size_t)mb * 16;
    REQUIRE((size_t)(wml - w0) >= slots * rows * c.D * 4, "part_o region short");
    REQUIRE((size_t)(wsp - wml) >= slots * rows * 2 * 4, "part_ml region short");
    REQUIRE((size_t)(wsp - w0) + (size_t)B * 4 <= ws_bytes, "split counts past the workspace");

    // the split target: one round of 256 workgroups per KV head (pairs of heads for a paired
    // drafting pass), or, for verification of at most kHostPlanMax sequences, whole rounds up to four
    {
        const int groups = (gather && a.pair) ? c.hkv / 2 : c.hkv;
        const int base = std::max(1, 256 / groups);
        REQUIRE(a.target % base == 0 && a.target >= base && a.target <= 4 * base, "target %d (round %d)", a.target,
                base);
        REQUIRE(a.target == base || (!gather && B <= vegas::kHostPlanMax), "target %d over one round", a.target);
        if (a.target > base) ++g_multiround;
    }
    std::vector<int> len, lo;
    spans(c, gather, len, lo);
    // the device plan: the grid (max_units per KV head) and the slots (nsplit)
    const DevPlan dp = device_plan(len, a.target, cap);
    for (int b = 0; b < B; ++b) {
        REQUIRE(dp.ns_raw[b] <= a.nsplit, "device plan: seq %d needs %d splits > nsplit %d", b, dp.ns_raw[b],
                a.nsplit);
        if (len[b] > 0) {
            REQUIRE(dp.chunk[b] <= cap, "device plan: seq %d chunk %d > cap %d", b, dp.chunk[b], cap);
            REQUIRE((long long)dp.ns_raw[b] * dp.chunk[b] >= len[b] && (long long)(dp.ns_raw[b] - 1) * dp.chunk[b] < len[b],
                    "device plan: seq %d splits %d x %d vs %d positions", b, dp.ns_raw[b], dp.chunk[b], len[b]);
        }
        if (page > 0 && !gather)
            for (int s = 0; s < dp.ns_raw[b]; ++s) {
                const int st = lo[b] + s * dp.chunk[b], en = std::min(st + dp.chunk[b], lo[b] + len[b]);
                REQUIRE(pages_spanned(st, en, page) <= a.page_cap, "device plan: %d pages > page list %d",
                        pages_spanned(st, en, page), a.page_cap);
            }
    }
    REQUIRE(dp.units <= a.max_units, "device plan: %lld units > max_units %d", dp.units, a.max_units);

    // LDS of the split kernel within the CU's 160 KB: its static arrays (the K/V ring, or the wave
    // merge's slots when larger: attn.hip's Geo, plus the staged index list of a gather pass and a
    // few words of plan state), then the dynamic collected-score buffer and a paged verification's
    // page list
    {
        const int db = c.D / 16;
        const int mslot = (db * mb * 4 + 2 * mb) * 64 * 4;
        const int ring = vegas::attn_ring_bytes(bf16, c.D, gather);
        const int main_lds = std::max(ring, (vegas::kAttnWaves / 2) * mslot);
        const long long stat = main_lds + (gather ? vegas::kMaxGatherChunk * 4 : 4) + 64;
        const long long dyn = (!gather && g_cap.collect ? vegas::attn_score_lds_bytes(a.score_cap) : 0) +
                              (!gather && page > 0 ? (long long)a.page_cap * 4 : 0);
        REQUIRE(stat + dyn <= 160 * 1024, "LDS %lld static + %lld dynamic", stat, dyn);
    }

    const vegas::HostPlan& hp = a.hp;
    // the collected-score LDS buffer (sized at launch) holds the longest unit
    if (!gather) {
        if (hp.n == 0) REQUIRE(a.score_cap == cap, "device plan: score buffer %d, cap %d", a.score_cap, cap);
        REQUIRE(a.score_cap <= cap, "score buffer %d above cap %d", a.score_cap, cap);
        // a unit's last block writes the collected scores of all its 16 positions (also those past
        // the unit's end): the buffer holds whole blocks
        REQUIRE(a.score_cap % vegas::kAttnBlock == 0, "score buffer %d not whole blocks", a.score_cap);
        if (hp.n > 0 && hp.nwg == 0)
            for (int b = 0; b < B; ++b)
                if (hp.first[b + 1] > hp.first[b])
                    REQUIRE(std::min(hp.chunk[b], hp.len[b]) <= a.score_cap, "seq %d split %d > score buffer %d", b,
                            std::min(hp.chunk[b], hp.len[b]), a.score_cap);
        if (hp.nwg > 0)
            for (int u = 0; u < hp.wg_first[hp.nwg]; ++u)
                REQUIRE(hp.u_end[u] - hp.u_start[u] <= a.score_cap, "unit %d longer than the score buffer %d", u,
                        a.score_cap);
    }
    if (hp.n == 0) return;
    REQUIRE(hp.n == B && B <= vegas::kHostPlanMax, "host plan over %d sequences", hp.n);
    if (hp.nwg == 0) {
        // the host plan must be the device plan, bit for bit
        for (int b = 0; b < B; ++b) {
            const int ns = hp.first[b + 1] - hp.first[b];
            REQUIRE(ns == std::min(dp.ns_raw[b], a.nsplit), "host/device split counts differ at seq %d", b);
            if (len[b] > 0) REQUIRE(hp.chunk[b] == dp.chunk[b], "host/device chunk differs at seq %d", b);
            REQUIRE(hp.len[b] == len[b] && hp.lo[b] == lo[b], "host span differs at seq %d", b);
        }
        REQUIRE(hp.first[0] == 0 && hp.first[B] <= a.max_units, "host grid %d", hp.first[B]);
        return;
    }
    // balanced plan
    ++g_balanced;
    REQUIRE(!gather, "balanced plan for a gather pass");
    REQUIRE(hp.nwg >= 1 && hp.nwg <= vegas::kHostWgMax, "nwg %d", hp.nwg);
    const int nu = hp.wg_first[hp.nwg];
    REQUIRE(hp.wg_first[0] == 0 && nu >= hp.nwg && nu <= vegas::kHostUnitsMax, "units %d", nu);
    std::vector<int> next_slot(B, 0), next_pos(B, 0);
    for (int b = 0; b < B; ++b) next_pos[b] = lo[b];
    for (int w = 0; w < hp.nwg; ++w) {
        REQUIRE(hp.wg_first[w + 1] >= hp.wg_first[w], "wg_first decreases at %d", w);
        for (int u = hp.wg_first[w]; u < hp.wg_first[w + 1]; ++u) {
            const int b = hp.u_bs[u] & 31, slot = hp.u_bs[u] >> 5;
            REQUIRE(b < B, "unit %d: sequence %d", u, b);
            REQUIRE(slot == next_slot[b] && slot < a.nsplit, "unit %d: slot %d (expected %d, nsplit %d)", u, slot,
                    next_slot[b], a.nsplit);
            REQUIRE(hp.u_start[u] == next_pos[b] && hp.u_end[u] > hp.u_start[u], "unit %d: [%d, %d) after %d", u,
                    hp.u_start[u], hp.u_end[u], next_pos[b]);
            REQUIRE(hp.u_end[u] - hp.u_start[u] <= cap, "unit %d: %d positions > cap %d", u,
                    hp.u_end[u] - hp.u_start[u], cap);
            ++next_slot[b];
            next_pos[b] = hp.u_end[u];
        }
    }
    for (int b = 0; b < B; ++b) {
        REQUIRE(next_pos[b] == lo[b] + len[b], "balanced plan leaves seq %d at %d of %d", b, next_pos[b],
                lo[b] + len[b]);
        REQUIRE(hp.first[b + 1] - hp.first[b] == next_slot[b], "first[] of seq %d", b);
    }
}

void check_select(const Case& c, size_t ws_bytes, size_t sel_offset, const char* entry) {
    const std::string ctx = c.ctx + " entry=" + entry;
    const vegas::SelectArgs& s = g_cap.s;
    REQUIRE(s.nchunks >= 0 && s.nchunks <= vegas::kSelMaxChunks, "nchunks %d", s.nchunks);
    const char* base = reinterpret_cast<const char*>(s.keys) - sel_offset;
    auto inside = [&](const void* p, size_t n) {
        const char* q = reinterpret_cast<const char*>(p);
        return q >= base && q + n <= base + ws_bytes;
    };
    REQUIRE(inside(s.keys, (size_t)c.total_kv * 4) && inside(s.cand_key, (size_t)c.total_kv * 4) &&
                inside(s.cand_pos, (size_t)c.total_kv * 4),
            "key buffers outside the workspace");
    REQUIRE(inside(s.zeroed, (size_t)vegas::select_zeroed_words(c.B) * 4), "histograms outside the workspace");
    REQUIRE(inside(s.seq_info, (size_t)c.B * 16) && inside(s.chunk_above, (size_t)c.B * s.nchunks * 4) &&
                inside(s.chunk_off, (size_t)c.B * s.nchunks * 4) && inside(s.chunk_ties, (size_t)c.B * s.nchunks * 4),
            "per-chunk tables outside the workspace");
    // longest prefix covered by the chunks
    const int W = c.gamma + 1;
    for (int b = 0; b < c.B; ++b) {
        const int L = c.cu[b + 1] - c.cu[b] - W;
        REQUIRE((long long)s.nchunks * vegas::kSelChunk >= L, "seq %d: %d chunks for %d positions", b, s.nchunks, L);
    }
    if (s.hg_n == 0) return;
    REQUIRE(s.hg_n == c.B && c.B <= vegas::kHostPlanMax, "selection geometry of %d sequences", s.hg_n);
    for (int b = 0; b < c.B; ++b) {
        const int L = c.cu[b + 1] - c.cu[b] - W;
        REQUIRE(s.hg_seq0[b] == c.cu[b] && s.hg_L[b] == L, "seq %d geometry", b);
        REQUIRE(s.hg_k[b] >= 0 && s.hg_k[b] <= s.hg_L[b], "seq %d: k %d of %d", b, s.hg_k[b], s.hg_L[b]);
        REQUIRE(s.hg_kout[b] == c.cuk[b] && s.hg_kout[b] + s.hg_k[b] <= c.cuk[c.B], "seq %d output slots", b);
    }
}

// One random batch.
Case make_case() {
    Case c;
    c.dtype = unif() < 0.75 ? VEGAS_DTYPE_BF16 : VEGAS_DTYPE_F32;
    c.D = unif() < 0.5 ? 64 : 128;
    static const int hkvs[] = {1, 2, 4, 8, 8, 8, 16};
    c.hkv = hkvs[uni(0, 6)];
    const int max_rows = (c.dtype == VEGAS_DTYPE_F32 && c.D == 128) ? 32 : 64;
    int G = 1 << uni(0, 3);
    while (G > max_rows) G >>= 1;
    c.hq = c.hkv * G;
    c.gamma = (int)uni(0, std::min(31, max_rows / G - 1));
    const int W = c.gamma + 1;
    // batch: mostly small, sometimes up to 1024
    const double rb = unif();
    c.B = rb < 0.6 ? (int)uni(1, 16) : rb < 0.9 ? (int)uni(17, 64) : (int)uni(65, 1024);
    // prefix lengths: equal, ragged log-uniform, tiny, mixed with empties, or
    // long and ragged (log-uniform over the top 5 octaves: balanced plans)
    const int mode = (int)uni(0, 4);
    const int64_t cap_total = 2000000000LL / std::max(1, c.B);
    const int64_t lmax = std::min<int64_t>(std::min<int64_t>(600000, cap_total), 4096LL * 2048 - W);
    std::vector<int> L(c.B);
    const int eq = (int)uni(0, lmax);
    for (int b = 0; b < c.B; ++b) {
        if (mode == 0) L[b] = eq;
        else if (mode == 1) L[b] = (int)std::exp(std::log(1.0) + unif() * std::log((double)lmax + 1.0)) - 1;
        else if (mode == 2) L[b] = (int)uni(0, 300);
        else if (mode == 3) L[b] = unif() < 0.3 ? 0 : (int)uni(0, lmax);
        else L[b] = (int)std::exp(std::log((double)lmax / 32 + 1) + unif() * std::log(32.0));
        L[b] = std::max(0, std::min<int>(L[b], (int)lmax));
    }
    c.cu.assign(c.B + 1, 0);
    c.cuk.assign(c.B + 1, 0);
    c.max_seqlen = 0;
    c.max_k = 0;
    const double ratio = unif() < 0.2 ? unif() : 0.05 + 0.1 * unif();
    for (int b = 0; b < c.B; ++b) {
        c.cu[b + 1] = c.cu[b] + L[b] + W;
        c.max_seqlen = std::max(c.max_seqlen, L[b] + W);
        const int k = std::min(L[b], (int)(ratio * L[b]));
        c.cuk[b + 1] = c.cuk[b] + k;
        c.max_k = std::max(c.max_k, k);
    }
    c.total_kv = c.cu[c.B];
    c.page = unif() < 0.3 ? (1 << uni(0, 8)) : 0;
    c.window = unif() < 0.2 ? (int)uni(1, 20000) : 0;
    char buf[256];
    std::snprintf(buf, sizeof buf, "case %lld: dtype=%d B=%d Hq=%d Hkv=%d D=%d gamma=%d page=%d window=%d maxL=%d",
                  g_cases, c.dtype, c.B, c.hq, c.hkv, c.D, c.gamma, c.page, c.window, c.max_seqlen);
    c.ctx = buf;
    return c;
}

void* fake(uintptr_t x) { return reinterpret_cast<void*>(x); }

void expect_ok(vegas_status_t st, const std::string& ctx, const char* entry) {
    if (st != VEGAS_OK)
        violation("entry point rejected valid arguments",
                  ctx + " entry=" + entry + " status=" + vegas_status_string(st) + ": " + vegas_last_error_message());
}

void run_case(const Case& c) {
    vegas_attn_shape_t shape{c.dtype, c.B, c.hq, c.hkv, c.D, 0.125f};
    const int es = c.dtype == VEGAS_DTYPE_BF16 ? 2 : 4;
    // contiguous caches whose rows would pass 32-bit byte offsets are rejected by design
    const bool contiguous_ok = (int64_t)c.max_seqlen * c.hkv * c.D * es < (int64_t(1) << 32);
    const vegas_host_offsets_t host{c.cu.data(), c.cuk.data()};
    void* q = fake(0x10000);
    void* kv = fake(0x20000);
    float* scores = static_cast<float*>(fake(0x30000));
    int32_t* idx = static_cast<int32_t*>(fake(0x40000));
    const int32_t* dcu = static_cast<const int32_t*>(fake(0x50000));
    const int32_t* dcuk = static_cast<const int32_t*>(fake(0x60000));
    void* out = fake(0x70000);
    const uint32_t mask = 1u | (1u << c.gamma);

    // verification (device and host plan), one-call verification + selection
    if (contiguous_ok && c.window == 0) {
        size_t vb = 0;
        expect_ok(vegas_verify_workspace_size(&shape, c.gamma, c.max_seqlen, &vb), c.ctx, "verify_workspace_size");
        void* ws = fake(0x100000000ULL);
        g_cap = Captured{};
        expect_ok(vegas_verify_attn(&shape, c.gamma, q, kv, kv, dcu, c.max_seqlen, c.total_kv, mask, scores, out, ws,
                                    vb, nullptr),
                  c.ctx, "verify_attn");
        check_attn(c, false, vb, "verify_attn");
        g_cap = Captured{};
        expect_ok(vegas_verify_attn_hostplan(&shape, c.gamma, q, kv, kv, dcu, c.max_seqlen, c.total_kv, mask, scores,
                                             out, ws, vb, nullptr, &host),
                  c.ctx, "verify_attn_hostplan");
        check_attn(c, false, vb, "verify_attn_hostplan");
        if (c.max_seqlen <= vegas::kSelMaxChunks * vegas::kSelChunk) {
            size_t fb = 0;
            expect_ok(vegas_verify_select_workspace_size(&shape, c.gamma, c.max_seqlen, c.total_kv, &fb), c.ctx,
                      "verify_select_workspace_size");
            g_cap = Captured{};
            expect_ok(vegas_verify_select_hostplan(&shape, c.gamma, q, kv, kv, dcu, c.max_seqlen, c.total_kv, mask,
                                                   dcuk, scores, idx, out, ws, fb, nullptr, &host),
                      c.ctx, "verify_select_hostplan");
            check_attn(c, false, vb, "verify_select_hostplan");
            {
                const std::string ctx = c.ctx;
                REQUIRE(g_cap.fused && g_cap.sel_tail, "one call without the fused selection");
            }
            const size_t off = (reinterpret_cast<const char*>(g_cap.s.keys) - static_cast<const char*>(ws));
            check_select(c, fb, off, "verify_select_hostplan");
            g_cap = Captured{};
            expect_ok(vegas_verify_select(&shape, c.gamma, q, kv, kv, dcu, c.max_seqlen, c.total_kv, mask, dcuk,
                                          scores, idx, out, ws, fb, nullptr),
                      c.ctx, "verify_select");
            check_attn(c, false, vb, "verify_select");
            check_select(c, fb, off, "verify_select");
            size_t sb = 0;
            expect_ok(vegas_select_workspace_size(c.B, c.hkv, c.gamma, c.max_seqlen, c.total_kv, &sb), c.ctx,
                      "select_workspace_size");
            g_cap = Captured{};
            expect_ok(vegas_select_topk(c.B, c.hkv, c.gamma, scores, dcu, c.max_seqlen, c.total_kv, dcuk, idx, ws, sb,
                                        nullptr),
                      c.ctx, "select_topk");
            {
                const std::string ctx = c.ctx;
                REQUIRE(g_cap.sel_full, "selection not launched");
            }
            check_select(c, sb, 0, "select_topk");
        }
    }
    if (contiguous_ok && c.window > 0) {
        size_t lb = 0;
        expect_ok(vegas_verify_local_workspace_size(&shape, c.gamma, c.max_seqlen, c.window, &lb), c.ctx,
                  "verify_local_workspace_size");
        g_cap = Captured{};
        expect_ok(vegas_verify_attn_local(&shape, c.gamma, q, kv, kv, dcu, c.max_seqlen, c.total_kv, c.window, out,
                                          fake(0x100000000ULL), lb, nullptr),
                  c.ctx, "verify_attn_local");
        check_attn(c, false, lb, "verify_attn_local");
    }
    // paged verification and drafting
    std::vector<int32_t> table(1, 0);
    if (c.page > 0) {
        const int maxp = (c.max_seqlen + c.page - 1) / c.page;
        const vegas_paged_kv_t pages{table.data(), maxp, c.page, std::max(1, c.total_kv / c.page + c.B)};
        if ((int64_t)pages.num_pages * c.page < (int64_t(1) << 31)) {
            size_t pb = 0;
            expect_ok(vegas_verify_paged_workspace_size(&shape, c.gamma, c.max_seqlen, c.page, &pb), c.ctx,
                      "verify_paged_workspace_size");
            g_cap = Captured{};
            Case cp = c;
            cp.window = 0;
            expect_ok(vegas_verify_attn_paged(&shape, c.gamma, q, kv, kv, &pages, dcu, c.max_seqlen, c.total_kv, mask,
                                              scores, out, fake(0x100000000ULL), pb, nullptr),
                      c.ctx, "verify_attn_paged");
            check_attn(cp, false, pb, "verify_attn_paged", c.page);
            size_t db = 0;
            expect_ok(vegas_sparse_decode_workspace_size(&shape, c.max_k, &db), c.ctx, "sparse_decode_workspace_size");
            g_cap = Captured{};
            expect_ok(vegas_sparse_decode_attn_paged(&shape, q, kv, kv, &pages, dcu, c.total_kv, idx, dcuk, c.max_k,
                                                     out, fake(0x100000000ULL), db, nullptr),
                      c.ctx, "sparse_decode_attn_paged");
            check_attn(c, true, db, "sparse_decode_attn_paged", c.page);
        }
    }
    // drafting (device and host plan)
    size_t db = 0;
    expect_ok(vegas_sparse_decode_workspace_size(&shape, c.max_k, &db), c.ctx, "sparse_decode_workspace_size");
    g_cap = Captured{};
    expect_ok(vegas_sparse_decode_attn(&shape, q, kv, kv, dcu, c.total_kv, idx, dcuk, c.max_k, out,
                                       fake(0x100000000ULL), db, nullptr),
              c.ctx, "sparse_decode_attn");
    check_attn(c, true, db, "sparse_decode_attn");
    g_cap = Captured{};
    expect_ok(vegas_sparse_decode_attn_hostplan(&shape, q, kv, kv, dcu, c.total_kv, idx, dcuk, c.max_k, out,
                                                fake(0x100000000ULL), db, nullptr, &host),
              c.ctx, "sparse_decode_attn_hostplan");
    check_attn(c, true, db, "sparse_decode_attn_hostplan");
}

}  // namespace

int main(int argc, char** argv) {
    const long long n = argc > 1 ? std::atoll(argv[1]) : 100000;
    const unsigned long long seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1;
    rng.seed(seed);
    for (g_cases = 0; g_cases < n; ++g_cases) run_case(make_case());
    std::printf("ok %lld cases, %lld balanced plans, %lld multi-round plans (seed %llu)\n", g_cases, g_balanced,
                g_multiround, seed);
    return 0;
}
