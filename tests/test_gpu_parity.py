"""GPU parity of the verify -> select -> sparse-draft path against the CPU oracle,
through the C ABI.  Every input is seeded and synthetic (workloads module)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from verification_guided_sparse_verify_amd import workloads as W
from verification_guided_sparse_verify_amd import vegas as V
from verification_guided_sparse_verify_amd.step import LayerStep

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from parity_util import ATOL, check_layer, log, run_layer


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def test_tiny_fp32_mqa_config():
    wl = W.named_workload(0)
    log(f"case: {wl.name}")
    inp, st = run_layer(wl, seed=0)
    worst = check_layer(wl, inp, st)
    log(f"  worst {worst}")
    assert wl.k_per_seq == [51]
    # The planted heavy hitters raise the collected score: the selection holds the same ones as the
    # oracle's, more than a random 5% selection would (0.5 of 10 on average, 3 or more with
    # probability ~1%); the device-drawn inputs of seed 0 give 3 of the 10.
    hh = set(W.heavy_hitter_positions(wl, seed=0)[0].tolist())
    t_gpu = set(st.indices[:51].cpu().tolist())
    q, k, v = (W.host_bits(inp[n]) for n in ("q", "k", "v"))
    cu = np.array(wl.cu_seqlens(), np.int32)
    _, s_ref = oracle.verify_attn(q, k, v, cu, wl.gamma, wl.scale)
    t_ref, _, _ = oracle.select_topk(s_ref, cu, wl.gamma, np.array(wl.cu_k(), np.int32))
    assert hh & t_gpu == hh & set(t_ref.tolist())
    assert len(hh & t_gpu) >= 3, sorted(hh & t_gpu)


SWEEP = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, ratio
    ("bf16", 1, 4, 4, 64, 0, [1], Fraction(5, 100)),
    ("bf16", 2, 4, 2, 64, 2, [0, 10], Fraction(1, 2)),
    ("bf16", 2, 8, 1, 128, 7, [63, 65], Fraction(5, 100)),
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], Fraction(5, 100)),
    ("f32", 2, 8, 2, 64, 2, [300, 77], Fraction(5, 100)),
    ("f32", 1, 4, 1, 128, 5, [513], Fraction(7, 100)),
    ("bf16", 2, 12, 4, 64, 4, [5000, 31], Fraction(5, 100)),
    ("bf16", 1, 64, 8, 128, 6, [2000], Fraction(10, 100)),
    ("bf16", 4, 32, 8, 128, 4, [3000, 1, 200, 9999], Fraction(5, 100)),
    ("bf16", 2, 16, 8, 64, 3, [777, 12000], Fraction(1)),
    # 40, 48 and 56 query rows per KV head: three and four row tiles held by one wave
    ("bf16", 2, 64, 8, 64, 4, [3000, 517], Fraction(5, 100)),
    ("f32", 1, 64, 8, 64, 6, [900], Fraction(5, 100)),
    ("bf16", 3, 64, 8, 128, 6, [5000, 64, 2047], Fraction(5, 100)),
    ("bf16", 2, 32, 4, 128, 4, [2500, 4100], Fraction(5, 100)),
    ("f32", 2, 32, 4, 64, 5, [1500, 33], Fraction(5, 100)),
    # drafting workgroups on one KV head: an odd KV head count, and 32 query rows per KV head
    # (two row tiles); the other cases above draft on KV head pairs
    ("bf16", 2, 12, 3, 64, 3, [2000, 513], Fraction(5, 100)),
    ("bf16", 2, 64, 2, 128, 1, [3000, 700], Fraction(5, 100)),
]


def test_kv_cache_pair_places_v_off_k():
    """The generator's device caches: K at a 2 MB boundary and V KV_GAP_BYTES + KV_OFFSET_BYTES past
    K's end rounded up to 2 MB, in one allocation, both contiguous, and the drawn values do not
    depend on the placement."""
    wl = W.custom_workload("bf16", 2, 8, 2, 128, 2, [3000, 700])
    inp = W.make_inputs(wl, seed=3, device="cuda:0")
    k, v = inp["k"], inp["v"]
    assert k.is_contiguous() and v.is_contiguous()
    assert k.data_ptr() % (2 << 20) == 0
    nbytes = k.numel() * k.element_size()
    kb = (nbytes + (2 << 20) - 1) // (2 << 20) * (2 << 20)
    assert v.data_ptr() - k.data_ptr() == kb + W.KV_GAP_BYTES + W.KV_OFFSET_BYTES
    assert k.untyped_storage().data_ptr() == v.untyped_storage().data_ptr()   # one allocation
    plain = {n: torch.empty_like(k) for n in ("k", "v")}           # two plain allocations
    ref = W.make_inputs(wl, seed=3, device="cuda:0", out=plain)
    assert ref["k"].data_ptr() == plain["k"].data_ptr()
    assert torch.equal(k, ref["k"]) and torch.equal(v, ref["v"])


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-L{c[6]}")
def test_shape_sweep(case):
    dtype, B, hq, hkv, d, gamma, prefixes, ratio = case
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, ratio=ratio)
    log(f"case: {wl.name} L={prefixes} ratio={ratio}")
    inp, st = run_layer(wl, seed=1)
    worst = check_layer(wl, inp, st)
    log(f"  worst {worst}")


def test_collection_toggle_leaves_output_bit_identical():
    """With collection off the kernel must compute plain attention ('Vegas ...', sec. 4)."""
    wl = W.custom_workload("bf16", 2, 32, 8, 128, 4, [3000, 1500])
    inp, st = run_layer(wl, seed=2)
    on = st.out.clone()
    st.verify(collect=False)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), st.out.view(torch.int16))


def test_repeat_runs_are_bitwise_deterministic():
    wl = W.custom_workload("bf16", 2, 32, 8, 128, 5, [6000, 2500])
    inp, st = run_layer(wl, seed=3)
    a = (st.out.clone(), st.scores.clone(), st.indices.clone(), st.draft_out.clone())
    st.run()
    torch.cuda.synchronize()
    b = (st.out, st.scores, st.indices, st.draft_out)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)


def test_sparse_full_list_equals_verification_row():
    """Sparse attention over every key row r sees equals verification row r."""
    wl = W.custom_workload("bf16", 2, 16, 4, 128, 3, [900, 2049])
    inp, st = run_layer(wl, seed=4)
    cu = wl.cu_seqlens()
    Wr = wl.gamma + 1
    for r in range(Wr):
        lists = [torch.arange(L + r + 1, dtype=torch.int32) for L in wl.prefix_lens]
        cui = torch.tensor([0, len(lists[0]), len(lists[0]) + len(lists[1])], dtype=torch.int32, device="cuda")
        idx = torch.cat(lists).cuda()
        q = torch.stack([inp["q"][b * Wr + r] for b in range(wl.batch)]).contiguous()
        out = torch.empty_like(q)
        mx = max(len(x) for x in lists)
        ws = torch.empty(V.vegas_sparse_decode_workspace_size(st.shape, mx), dtype=torch.uint8, device="cuda")
        V.vegas_sparse_decode_attn(st.shape, q, inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv, idx, cui, mx,
                                   out, ws)
        torch.cuda.synchronize()
        ref = torch.stack([st.out[b * Wr + r] for b in range(wl.batch)])
        err = (out.float() - ref.float()).abs().max().item()
        assert err <= 2e-2, f"row {r}: {err}"


def test_all_zero_queries_select_lowest_positions():
    """Q = 0 makes every collected score 0: the tie rule takes positions 0..k-1."""
    wl = W.custom_workload("bf16", 2, 8, 2, 64, 2, [5000, 700])
    inp = W.make_inputs(wl, seed=5, device="cuda")
    inp["q"].zero_()
    inp, st = run_layer(wl, inputs=inp)
    cuk = wl.cu_k()
    for b in range(wl.batch):
        got = st.indices[cuk[b]:cuk[b + 1]].cpu().tolist()
        assert got == list(range(wl.k_per_seq[b]))


LOGIT_CASES = [
    ("bf16", 128, "drift"), ("bf16", 64, "drift"), ("bf16", 128, "wide"), ("f32", 64, "drift"),
]


@pytest.mark.parametrize("case", LOGIT_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-{c[2]}")
def test_logit_patterns_that_move_the_softmax_reference(case):
    """Logits with a designed course along the positions, so the kernels' running softmax
    reference moves often: 'drift' oscillates by +-7 (log2 units) around a rise of 12 over the
    prefix, so many blocks carry weight and the reference moves a few times; 'wide' draws
    every position's logit with a spread of 40 (log2 units), so it moves many times early.
    Built as K = f(pos)/D * u_g + small noise and q = a * u_g (u_g a +-1 vector per KV head,
    a per row and head in [0.8, 1.2])."""
    dt, d, pattern = case
    wl = W.custom_workload(dt, 2, 8, 2, d, 3, [3000, 1200], plants=False)
    inp = W.make_inputs(wl, seed=21, device="cuda")
    g = torch.Generator().manual_seed(77)
    tdt = inp["k"].dtype
    log2e = 1.4426950408889634
    u = torch.randint(0, 2, (wl.num_kv_heads, d), generator=g).double() * 2 - 1
    cu = wl.cu_seqlens()
    k = torch.empty(wl.total_kv, wl.num_kv_heads, d, dtype=torch.float64)
    for b in range(wl.batch):
        n = cu[b + 1] - cu[b]
        pos = torch.arange(n, dtype=torch.float64)
        for h in range(wl.num_kv_heads):
            if pattern == "drift":
                t = 7.0 * torch.sin(2 * np.pi * pos / 200.0 + h) + 12.0 * pos / n
            else:
                t = 40.0 * torch.randn(n, generator=g, dtype=torch.float64)
            f = t / (wl.scale * log2e)
            k[cu[b]:cu[b + 1], h] = f[:, None] / d * u[h][None, :] + 0.02 * torch.randn(n, d, generator=g,
                                                                                        dtype=torch.float64)
    inp["k"].copy_(k.to(tdt))
    G = wl.num_q_heads // wl.num_kv_heads
    heads = torch.arange(wl.num_q_heads) // G
    qa = 0.8 + 0.4 * torch.rand(wl.batch * (wl.gamma + 1), wl.num_q_heads, 1, generator=g, dtype=torch.float64)
    inp["q"].copy_((qa * u[heads][None]).to(tdt))
    da = 0.8 + 0.4 * torch.rand(wl.n_drafts, wl.batch, wl.num_q_heads, 1, generator=g, dtype=torch.float64)
    inp["draft_q"].copy_((da * u[heads][None, None]).to(tdt))
    inp, st = run_layer(wl, inputs=inp)
    worst = check_layer(wl, inp, st)
    log(f"{dt} D{d} {pattern}: {worst}")


def test_empty_draft_list_gives_zero_rows():
    wl = W.custom_workload("bf16", 2, 8, 2, 128, 1, [100, 100])
    inp = W.make_inputs(wl, seed=6, device="cuda")
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale)
    cui = torch.tensor([0, 0, 3], dtype=torch.int32, device="cuda")
    idx = torch.tensor([5, 50, 99], dtype=torch.int32, device="cuda")
    out = torch.full_like(inp["draft_q"][0], 7.0)
    V.vegas_sparse_decode_attn(st.shape, inp["draft_q"][0], inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv,
                               idx, cui, 3, out, st.workspace)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0)
    dq = W.host_bits(inp["draft_q"][0])
    ref = oracle.sparse_decode_attn(dq, W.host_bits(inp["k"]), W.host_bits(inp["v"]),
                                    wl.cu_seqlens(), idx.cpu().numpy(), cui.cpu().numpy(), wl.scale)
    assert np.abs(out.float().cpu().numpy() - ref).max() <= 2e-2


def test_all_draft_lists_empty():
    """Every list empty (nothing to gather anywhere): all rows are zero."""
    wl = W.custom_workload("bf16", 3, 8, 2, 128, 1, [100, 40, 7])
    inp = W.make_inputs(wl, seed=7, device="cuda")
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale)
    cui = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    for max_idx in (0, 5):
        out = torch.full_like(inp["draft_q"][0], 7.0)
        V.vegas_sparse_decode_attn(st.shape, inp["draft_q"][0], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                   wl.total_kv, idx, cui, max_idx, out, st.workspace)
        torch.cuda.synchronize()
        assert torch.all(out == 0)


def _draft_case():
    """Two sequences whose lists take many splits per KV head (many partials to merge)."""
    wl = W.custom_workload("bf16", 2, 16, 4, 128, 2, [20000, 9000], ratio=Fraction(20, 100))
    inp, st = run_layer(wl, seed=8)
    return wl, inp, st


def test_draft_merge_takes_any_workspace_contents():
    """The drafting call needs nothing from the workspace's previous contents: zeros, all ones,
    random bytes and another call's leftovers give the same bits."""
    wl, inp, st = _draft_case()
    ref = st.draft_out[0].clone()
    gen = torch.Generator(device="cuda").manual_seed(0)
    fills = [lambda w: w.zero_(), lambda w: w.fill_(255),
             lambda w: w.copy_(torch.randint(0, 256, w.shape, generator=gen, device="cuda", dtype=torch.uint8)),
             lambda w: st.verify()]
    for fill in fills:
        fill(st.workspace)
        out = torch.full_like(ref, 3.0)
        V.vegas_sparse_decode_attn(st.shape, inp["draft_q"][0], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                   wl.total_kv, st.indices, inp["cu_k"], st.max_k, out, st.workspace)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    check_layer(wl, inp, st)


def test_draft_graph_replays():
    """A drafting call captured in a HIP graph gives the eager result on every replay, also after
    eager calls on the same workspace in between."""
    wl, inp, st = _draft_case()
    ref = st.draft_out[1].clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up outside the capture
        V.vegas_sparse_decode_attn(st.shape, inp["draft_q"][1], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                   wl.total_kv, st.indices, inp["cu_k"], st.max_k, out, st.workspace)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        V.vegas_sparse_decode_attn(st.shape, inp["draft_q"][1], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                   wl.total_kv, st.indices, inp["cu_k"], st.max_k, out, st.workspace)
    for rep in range(4):
        out.fill_(5.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        if rep == 1:                    # eager calls on the same workspace in between
            st.draft(0)
            st.draft(1)
            torch.cuda.synchronize()


def test_qwen3_8b_layer_full():
    wl = W.named_workload(1)
    log(f"case: {wl.name}")
    inp, st = run_layer(wl, seed=0)
    worst = check_layer(wl, inp, st)
    log(f"  worst {worst}")


def test_gpt_oss_ragged_sampled():
    wl = W.named_workload(4)
    log(f"case: {wl.name} prefixes={wl.prefix_lens}")
    inp, st = run_layer(wl, seed=0)
    order = np.argsort(wl.prefix_lens)
    seqs = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    worst = check_layer(wl, inp, st, seqs=seqs)
    log(f"  sequences {seqs} worst {worst}")


def test_largest_batch_and_row_count():
    """The largest batch the attention passes plan (1024 sequences, ragged, some empty) with the
    largest query-row count per KV head (gamma 31 at GQA group 2: 64 rows, the row-split path)."""
    rng = np.random.default_rng(11)
    prefixes = [int(x) for x in rng.integers(0, 300, size=1024)]
    prefixes[0], prefixes[1], prefixes[-1] = 0, 1, 299
    wl = W.custom_workload("bf16", 1024, 16, 8, 64, 31, prefixes, draft_steps=2)
    log(f"case: {wl.name} (1024 ragged sequences, 64 rows per KV head)")
    inp, st = run_layer(wl, seed=4)
    seqs = sorted({0, 1, 2, 511, 1022, 1023} | {int(x) for x in rng.integers(0, 1024, size=10)})
    worst = check_layer(wl, inp, st, seqs=seqs)
    log(f"  sequences {seqs} worst {worst}")
    # every list is valid: k_b distinct ascending prefix positions
    idx, cuk = st.indices.cpu().numpy(), wl.cu_k()
    for b in range(1024):
        t = idx[cuk[b]:cuk[b + 1]]
        assert len(t) == wl.k_per_seq[b]
        assert np.all(np.diff(t) > 0) and (len(t) == 0 or (t[0] >= 0 and t[-1] < prefixes[b])), b


def test_qwen3_32b_clustered_sampled():
    wl = W.named_workload(3)
    log(f"case: {wl.name}")
    inp, st = run_layer(wl, seed=0)
    worst = check_layer(wl, inp, st, seqs=[0, 5])
    log(f"  worst {worst}")


def test_qwen3_8b_128k_layer_sampled():
    """One layer of the 128K decode step (per-layer seed), one sequence checked in full."""
    wl = W.named_workload(2)
    log(f"case: {wl.name} (layer 7)")
    inp, st = run_layer(wl, seed=0, layer=7)
    worst = check_layer(wl, inp, st, seqs=[2])
    log(f"  worst {worst}")


SELECT_CASES = [
    # KV heads, gamma, prefix lengths, k per sequence, integer score range (ties)
    (2, 3, [5000, 70000, 1], [250, 3500, 1], 3),
    (8, 5, [131072, 40000], [6553, 40000], 2),
    (1, 0, [2049, 2047, 4096], [1, 2047, 0], 1),
    (4, 1, [300000], [15000], 0),
    # more ragged and tie-heavy lists: a partial last chunk, k = L, k = 1, all scores equal
    (2, 3, [32768, 100, 0], [1638, 100, 0], 2),
    (2, 3, [32769, 5], [3000, 5], 2),
    (4, 1, [20000, 7], [1000, 7], 0),
    (3, 2, [4000, 31, 1], [3999, 1, 1], 1),
    # 128 and 129 chunks of 2048 positions; all-tied scores over more than 8192 positions
    (2, 3, [262140, 1000], [13107, 50], 2),
    (2, 3, [262141, 77], [13000, 3], 1),
    (1, 0, [9000, 30000], [4500, 29000], 0),
]


@pytest.mark.parametrize("case", SELECT_CASES, ids=lambda c: f"H{c[0]}-g{c[1]}-L{c[2]}-k{c[3]}-r{c[4]}")
def test_select_exact_on_tied_integer_scores(case):
    """Integer-valued scores sum exactly in fp32 and fp64, so the selected lists must
    equal the oracle's bit for bit, ties going to the lower position."""
    hkv, gamma, prefixes, ks, rng_r = case
    log(f"case: select hkv={hkv} gamma={gamma} L={prefixes} k={ks} range={rng_r}")
    W_ = gamma + 1
    lens = [L + W_ for L in prefixes]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    total = int(cu[-1])
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    if rng_r == 0:
        sc = torch.zeros(hkv, total, dtype=torch.float32)
    else:
        sc = torch.randint(-rng_r, rng_r + 1, (hkv, total), generator=g).to(torch.float32)
    idx_ref, _, _ = oracle.select_topk(sc.numpy().astype(np.float64), cu, gamma, cuk)
    dev = sc.cuda()
    out = torch.full((max(int(cuk[-1]), 1),), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(V.vegas_select_workspace_size(len(prefixes), hkv, gamma, max(lens), total),
                     dtype=torch.uint8, device="cuda")
    V.vegas_select_topk(len(prefixes), hkv, gamma, dev, torch.from_numpy(cu).cuda(), max(lens), total,
                        torch.from_numpy(cuk).cuda(), out, ws)
    torch.cuda.synchronize()
    got = out[: int(cuk[-1])].cpu().numpy()
    assert np.array_equal(got, idx_ref)


MASK_CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, collect mask (None: Collect-2-Query)
    ("bf16", 2, 32, 8, 128, 5, [3000, 700], "all"),
    ("bf16", 2, 16, 8, 64, 7, [1500, 2049], 0b10110010),
    ("f32", 1, 8, 2, 64, 3, [900], "all"),
    ("bf16", 3, 8, 1, 128, 2, [130, 1, 4100], 0b010),
    ("bf16", 1, 64, 8, 128, 6, [2500], "all"),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-m{c[7]}")
def test_collect_mask_variants(case):
    """Collection of any set of verification rows (all rows, as in the pages' first design;
    or an arbitrary subset): scores, selection and drafts match the oracle."""
    dtype, B, hq, hkv, d, gamma, prefixes, mask = case
    if mask == "all":
        mask = (1 << (gamma + 1)) - 1
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes)
    log(f"case: {wl.name} L={prefixes} mask={mask:#x}")
    inp, st = run_layer(wl, seed=8, collect_mask=mask)
    worst = check_layer(wl, inp, st, collect_mask=mask)
    log(f"  worst {worst}")


PAGED_CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, page size
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], 16),
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], 1),
    ("bf16", 2, 32, 8, 64, 5, [3000, 40], 256),
    ("f32", 2, 8, 2, 64, 2, [300, 77], 4),
    ("bf16", 1, 64, 8, 128, 6, [2000], 32),
    # 1-token pages with splits of ~3K positions, longer than a 2048-word page list alone would allow
    ("bf16", 1, 32, 8, 128, 3, [100000], 1),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-P{c[7]}")
def test_paged_cache_matches_contiguous(case):
    """The paged entry points read the same logical K/V through a block table, so verification,
    the scores, the selection and the drafts equal the contiguous path bit for bit (same splits,
    same arithmetic), and hence the oracle."""
    dtype, B, hq, hkv, d, gamma, prefixes, P = case
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes)
    log(f"case: paged {wl.name} L={prefixes} page={P}")
    inp, st = run_layer(wl, seed=9)
    pg = W.page_cache(wl, inp, P, seed=9)
    pages = V.paged_kv(pg["block_table"], P, pg["num_pages"])
    out = torch.empty_like(st.out)
    scores = torch.empty_like(st.scores)
    ws = torch.empty(max(V.vegas_verify_paged_workspace_size(st.shape, gamma, st.max_seqlen, P), st.workspace.numel()),
                     dtype=torch.uint8, device="cuda")
    V.vegas_verify_attn_paged(st.shape, gamma, inp["q"], pg["k_pool"], pg["v_pool"], pages, inp["cu_seqlens_k"],
                              st.max_seqlen, st.total_kv, st.collect_mask, scores, out, ws)
    idx = torch.empty_like(st.indices)
    V.vegas_select_topk(B, hkv, gamma, scores, inp["cu_seqlens_k"], st.max_seqlen, st.total_kv, inp["cu_k"], idx, ws)
    drafts = torch.empty_like(st.draft_out)
    for j in range(wl.n_drafts):
        V.vegas_sparse_decode_attn_paged(st.shape, inp["draft_q"][j], pg["k_pool"], pg["v_pool"], pages,
                                         inp["cu_seqlens_k"], st.total_kv, idx, inp["cu_k"], st.max_k, drafts[j], ws)
    torch.cuda.synchronize()
    cu = wl.cu_seqlens()
    assert torch.equal(out.view(torch.uint8), st.out.view(torch.uint8))
    for b in range(B):   # scores are defined on prefix positions only
        s0, L = cu[b], wl.prefix_lens[b]
        assert torch.equal(scores[:, s0:s0 + L], st.scores[:, s0:s0 + L])
    assert torch.equal(idx[: wl.cu_k()[-1]], st.indices[: wl.cu_k()[-1]])
    assert torch.equal(drafts.view(torch.uint8), st.draft_out.view(torch.uint8))
    check_layer(wl, inp, st)   # and the contiguous path against the oracle


MULTI_ROUND_CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, page size (0: contiguous)
    # 16 KV heads: one round is 16 splits per head; 400K positions need 17 of at most 24576
    ("bf16", 1, 16, 16, 64, 1, [400000], 0),
    # 1-token pages: the page list shares the split's LDS (13248 positions), 250K need 19 splits
    ("bf16", 1, 32, 16, 64, 3, [250000], 1),
]


@pytest.mark.parametrize("case", MULTI_ROUND_CASES, ids=lambda c: f"{c[0]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-L{c[6]}-P{c[7]}")
def test_multi_round_plans_match_oracle(case):
    """When the LDS cap forces more splits than one round of workgroups holds, the plan takes
    whole rounds (here two, twice the one-round split count); verification, scores, selection and
    drafts still match the oracle."""
    dtype, B, hq, hkv, d, gamma, prefixes, P = case
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, draft_steps=2)
    log(f"case: multi-round {wl.name} L={prefixes} page={P}")
    inp = W.make_inputs(wl, seed=12, device="cuda")
    paged = W.page_cache(wl, inp, P, seed=12) if P else None
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts, paged=paged)
    st.run()
    torch.cuda.synchronize()
    worst = check_layer(wl, inp, st)
    log(f"  worst {worst}")


LOCAL_CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, window
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], 128),
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], 1),
    ("bf16", 2, 64, 8, 64, 3, [20000, 50], 128),
    ("f32", 2, 8, 2, 64, 2, [300, 77], 64),
    ("bf16", 1, 32, 8, 128, 5, [700], 5000),
    ("bf16", 2, 64, 8, 128, 6, [3000, 40], 256),
]


@pytest.mark.parametrize("case", LOCAL_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-w{c[7]}")
def test_local_window_verify_matches_oracle(case):
    """Banded verification (row r sees keys L+r-window < j <= L+r) against the oracle."""
    dtype, B, hq, hkv, d, gamma, prefixes, window = case
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes)
    log(f"case: local {wl.name} L={prefixes} window={window}")
    inp = W.make_inputs(wl, seed=10, device="cuda")
    shape = V.attn_shape(V.VEGAS_DTYPE_BF16 if dtype == "bf16" else V.VEGAS_DTYPE_F32, B, hq, hkv, d, wl.scale)
    out = torch.empty_like(inp["q"])
    ws = torch.empty(V.vegas_verify_local_workspace_size(shape, gamma, max(wl.seqlens), window),
                     dtype=torch.uint8, device="cuda")
    V.vegas_verify_attn_local(shape, gamma, inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"], max(wl.seqlens),
                              wl.total_kv, window, out, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.verify_attn(W.host_bits(inp["q"]), W.host_bits(inp["k"]), W.host_bits(inp["v"]),
                                wl.cu_seqlens(), gamma, wl.scale, want_scores=False, window=window)
    err = float(np.abs(out.float().cpu().numpy() - ref).max())
    log(f"  max abs err {err}")
    assert err <= ATOL[dtype]


def test_streaming_lists_and_drafts_match_oracle():
    """Sink-plus-recent lists with the Vegas budget are bit-exact, and drafting over them matches."""
    wl = W.custom_workload("bf16", 3, 32, 8, 128, 4, [6000, 300, 2049])
    inp = W.make_inputs(wl, seed=11, device="cuda")
    cuk = wl.cu_k()
    idx = torch.full((cuk[-1],), -1, dtype=torch.int32, device="cuda")
    V.vegas_streaming_indices(wl.batch, wl.gamma, 4, inp["cu_seqlens_k"], wl.total_kv, inp["cu_k"], cuk[-1], idx)
    torch.cuda.synchronize()
    ref = oracle.streaming_indices(wl.cu_seqlens(), wl.gamma, 4, cuk)
    assert np.array_equal(idx.cpu().numpy(), ref)
    shape = V.attn_shape(V.VEGAS_DTYPE_BF16, wl.batch, 32, 8, 128, wl.scale)
    out = torch.empty_like(inp["draft_q"][0])
    ws = torch.empty(V.vegas_sparse_decode_workspace_size(shape, max(wl.k_per_seq)), dtype=torch.uint8, device="cuda")
    V.vegas_sparse_decode_attn(shape, inp["draft_q"][0], inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv, idx,
                               inp["cu_k"], max(wl.k_per_seq), out, ws)
    torch.cuda.synchronize()
    d_ref = oracle.sparse_decode_attn(W.host_bits(inp["draft_q"][0]), W.host_bits(inp["k"]), W.host_bits(inp["v"]),
                                      wl.cu_seqlens(), ref, cuk, wl.scale)
    assert np.abs(out.float().cpu().numpy() - d_ref).max() <= 2e-2


ACCEPT_CASES = [
    # batch, gamma, vocab, draft noise, temperature
    (4, 5, 151936, 0.6, 1.0),      # Qwen3 vocabulary
    (16, 3, 201088, 1.5, 0.6),     # gpt-oss vocabulary, sharper and less aligned drafts
    (8, 0, 5000, 0.0, 1.0),        # nothing drafted: the bonus token only
    (32, 7, 17, 0.3, 0.2),         # tiny vocabulary: exact ties and zero masses
]


@pytest.mark.parametrize("case", ACCEPT_CASES, ids=lambda c: f"B{c[0]}-g{c[1]}-V{c[2]}")
def test_spec_accept_bit_exact(case):
    """Accepted counts and emitted tokens equal the oracle's exactly (the decision arithmetic
    is order-independent by construction)."""
    B, gamma, Vsz, noise, temp = case
    log(f"case: accept B={B} gamma={gamma} V={Vsz}")
    inp = W.make_accept_inputs(B, gamma, Vsz, seed=12, device="cuda", draft_noise=noise, temperature=temp)
    n = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    t = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    V.vegas_spec_accept(B, gamma, Vsz, inp["p"], inp["q"] if gamma else None, inp["draft"] if gamma else None,
                         inp["u_accept"] if gamma else None, inp["u_sample"], n, t)
    torch.cuda.synchronize()
    h = {k: v.cpu().numpy() for k, v in inp.items()}
    n_ref, t_ref = oracle.spec_accept(h["p"], h["q"], h["draft"], h["u_accept"], h["u_sample"])
    log(f"  accepted {n.cpu().tolist()[:8]}")
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert np.array_equal(t.cpu().numpy(), t_ref)


def test_spec_accept_greedy_and_forced_rejections():
    """One-hot rows (greedy decoding) and drafts forced out by u = 1: the decision and the
    residual draw match the oracle."""
    B, gamma, Vv = 64, 4, 1000
    g = torch.Generator().manual_seed(13)
    tgt = torch.randint(0, Vv, (B, gamma + 1), generator=g)
    draft = torch.where(torch.rand(B, gamma, generator=g) < 0.6, tgt[:, :gamma],
                        torch.randint(0, Vv, (B, gamma), generator=g)).to(torch.int32)
    p = torch.zeros(B, gamma + 1, Vv)
    p.scatter_(2, tgt[..., None], 1.0)
    q = torch.softmax(torch.randn(B, gamma, Vv, generator=g), dim=-1)
    q.scatter_(2, draft.long()[..., None], 0.9)
    ua = torch.ones(B, gamma) * torch.rand(B, 1, generator=g)
    us = torch.rand(B, generator=g)
    dev = {k: v.contiguous().cuda() for k, v in dict(p=p, q=q, d=draft, ua=ua, us=us).items()}
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    t = torch.empty(B, dtype=torch.int32, device="cuda")
    V.vegas_spec_accept(B, gamma, Vv, dev["p"], dev["q"], dev["d"], dev["ua"], dev["us"], n, t)
    torch.cuda.synchronize()
    n_ref, t_ref = oracle.spec_accept(p.numpy(), q.numpy(), draft.numpy(), ua.numpy(), us.numpy())
    assert np.array_equal(n.cpu().numpy(), n_ref) and np.array_equal(t.cpu().numpy(), t_ref)


FUSED_CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, ratio
    ("bf16", 3, 16, 4, 128, 3, [1000, 4097, 129], Fraction(5, 100)),
    ("f32", 2, 8, 2, 64, 2, [300, 77], Fraction(5, 100)),
    ("bf16", 2, 16, 8, 64, 3, [777, 12000], Fraction(1)),
    ("bf16", 2, 4, 2, 64, 2, [0, 10], Fraction(1, 2)),
    ("bf16", 4, 32, 8, 128, 4, [3000, 1, 200, 9999], Fraction(5, 100)),
    ("bf16", 1, 64, 8, 128, 6, [2000], Fraction(10, 100)),
    "gpt-oss-ragged",
]


@pytest.mark.parametrize("case", FUSED_CASES,
                         ids=lambda c: c if isinstance(c, str) else f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-L{c[6]}")
def test_verify_select_one_call_equals_two_calls(case):
    """vegas_verify_select gives the outputs, scores and selection of vegas_verify_attn followed
    by vegas_select_topk bit for bit, whatever its workspace held before (its histograms are
    cleared inside the call), twice in a row."""
    if isinstance(case, str):
        wl = W.named_workload(4)
    else:
        dtype, B, hq, hkv, d, gamma, prefixes, ratio = case
        wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, ratio=ratio)
    log(f"case: one-call verify+select {wl.name}")
    inp, st = run_layer(wl, seed=5)
    cu, cuk = wl.cu_seqlens(), wl.cu_k()
    ws = torch.full((V.vegas_verify_select_workspace_size(st.shape, wl.gamma, st.max_seqlen, st.total_kv),),
                    0xA5, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        out = torch.empty_like(st.out)
        scores = torch.full_like(st.scores, float("nan"))
        idx = torch.full_like(st.indices, -7)
        V.vegas_verify_select(st.shape, wl.gamma, inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"], st.max_seqlen,
                              st.total_kv, st.collect_mask, inp["cu_k"], scores, idx, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), st.out.view(torch.uint8)), rep
        for b in range(wl.batch):
            s0, L = cu[b], wl.prefix_lens[b]
            assert torch.equal(scores[:, s0:s0 + L], st.scores[:, s0:s0 + L]), (rep, b)
        assert torch.equal(idx[: cuk[-1]], st.indices[: cuk[-1]]), rep
        ws.fill_(0xFF if rep == 0 else 0x00)
    if not isinstance(case, str):
        check_layer(wl, inp, st)


def test_out_of_range_device_indices_are_clamped():
    """Index values read from device memory are clamped to the owning sequence (the header's
    promise): a draft list holding negative and too-large positions attends to the clamped
    rows, as the oracle does on the clamped list; a selection budget above L_b writes the
    L_b prefix positions and leaves the extra slots alone."""
    from parity_util import _seq_host
    wl = W.custom_workload("bf16", 2, 16, 4, 64, 2, [300, 41])
    inp, st = run_layer(wl, seed=12)
    Wr = wl.gamma + 1
    lens = wl.seqlens
    raw = [np.array([-3, 5, 7, lens[0] + 50, 2 ** 30, 0], np.int32), np.array([lens[1], -1, 40, 9], np.int32)]
    clamped = [np.clip(x, 0, n - 1).astype(np.int32) for x, n in zip(raw, lens)]
    cui = np.array([0, len(raw[0]), len(raw[0]) + len(raw[1])], np.int32)
    q = inp["draft_q"][0].contiguous()
    out = torch.empty_like(q)
    mx = max(len(x) for x in raw)
    ws = torch.empty(V.vegas_sparse_decode_workspace_size(st.shape, mx), dtype=torch.uint8, device="cuda")
    V.vegas_sparse_decode_attn(st.shape, q, inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv,
                               torch.from_numpy(np.concatenate(raw)).cuda(), torch.from_numpy(cui).cuda(), mx, out, ws)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        _, k, v, cu1 = _seq_host(inp, wl, b)
        ref = oracle.sparse_decode_attn(W.host_bits(q[b:b + 1]), k, v, cu1, clamped[b],
                                        np.array([0, len(clamped[b])], np.int32), wl.scale)
        err = float(np.abs(out[b:b + 1].float().cpu().numpy() - ref).max())
        assert err <= ATOL["bf16"], (b, err)

    # selection budget above the prefix: k_0 = L_0 + 5
    L0, L1 = wl.prefix_lens
    cuk = np.array([0, L0 + 5, L0 + 5 + 3], np.int32)
    idx = torch.full((int(cuk[-1]),), -9, dtype=torch.int32, device="cuda")
    sws = torch.empty(V.vegas_select_workspace_size(wl.batch, wl.num_kv_heads, wl.gamma, max(lens), wl.total_kv),
                      dtype=torch.uint8, device="cuda")
    V.vegas_select_topk(wl.batch, wl.num_kv_heads, wl.gamma, st.scores, inp["cu_seqlens_k"], max(lens), wl.total_kv,
                        torch.from_numpy(cuk).cuda(), idx, sws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert np.array_equal(got[:L0], np.arange(L0))          # every prefix position, ascending
    assert np.all(got[L0:L0 + 5] == -9)                       # the extra slots untouched
    assert len(set(got[L0 + 5:].tolist())) == 3 and np.all(np.diff(got[L0 + 5:]) > 0)


HOSTPLAN_CASES = FUSED_CASES + [
    # equal lengths over several sequences (the 128K workload's shape, shorter)
    ("bf16", 4, 32, 8, 128, 5, [5000] * 4, Fraction(5, 100)),
    # 17 sequences: above the host plan's batch limit, planned on the device (same results)
    ("bf16", 17, 8, 2, 128, 2, [100 * (i + 1) for i in range(17)], Fraction(5, 100)),
    # a sequence whose list is empty next to non-empty ones
    ("bf16", 3, 8, 2, 128, 2, [5000, 10, 3000], Fraction(5, 100)),
    # ragged lengths for which the host balances the verification splits over the batch
    ("bf16", 12, 64, 8, 64, 3, [1705, 6093, 6444, 35657, 19991, 18445, 12287, 1781, 29032, 4948, 8582, 1443],
     Fraction(5, 100)),
    ("f32", 12, 32, 8, 64, 3, [2361, 4845, 2222, 5051, 10012, 14071, 2837, 4297, 2075, 28095, 3332, 37128],
     Fraction(5, 100)),
    # the same balancing with four row tiles per KV head (56 rows)
    ("bf16", 12, 64, 8, 128, 6, [1705, 6093, 6444, 35657, 19991, 18445, 12287, 1781, 29032, 4948, 8582, 1443],
     Fraction(5, 100)),
]


@pytest.mark.parametrize("case", HOSTPLAN_CASES,
                         ids=lambda c: c if isinstance(c, str) else f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}")
def test_hostplan_calls_equal_device_planned_calls(case):
    """The *_hostplan entry points (split plan from host copies of the offsets) against the entry
    points that plan on the device: collected scores, selections and drafting outputs bit for bit;
    verification outputs bit for bit unless the host balances a ragged batch's splits (asked of the
    library, vegas_verify_hostplan_info), which changes only the merge's rounding: then within the
    output tolerance; and everything matches the oracle."""
    if isinstance(case, str):
        wl = W.named_workload(4)
    else:
        dtype, B, hq, hkv, d, gamma, prefixes, ratio = case
        wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, ratio=ratio)
    log(f"case: host plan {wl.name}")
    inp = W.make_inputs(wl, seed=9, device="cuda")
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts)
    cu, cuk = wl.cu_seqlens(), wl.cu_k()

    def snapshot():
        torch.cuda.synchronize()
        return (st.out.clone(), [st.scores[:, cu[b]:cu[b] + wl.prefix_lens[b]].clone() for b in range(wl.batch)],
                st.indices[: cuk[-1]].clone(), st.draft_out.clone())

    st.run(fused=True)
    ref = snapshot()
    st.out.fill_(3.0)
    st.scores.fill_(float("nan"))
    st.indices.fill_(-7)
    st.draft_out.fill_(5.0)
    st.run(fused=True, host_plan=True)
    got = snapshot()
    balanced, _ = V.vegas_verify_hostplan_info(st.shape, wl.gamma, st.max_seqlen, st.total_kv, st.host)
    log(f"  balanced plan: {balanced}")
    if len(set(wl.seqlens)) == 1:
        assert not balanced

    def same_out(x, y):
        if not balanced:
            return torch.equal(x.view(torch.uint8), y.view(torch.uint8))
        return (x.float() - y.float()).abs().max().item() <= ATOL[wl.dtype]
    assert same_out(got[0], ref[0])
    for a, b in zip(got[1], ref[1]):
        assert torch.equal(a, b)
    assert torch.equal(got[2], ref[2])
    assert torch.equal(got[3][: wl.n_drafts].view(torch.uint8), ref[3][: wl.n_drafts].view(torch.uint8))
    for collect in (False, True):
        st.verify(collect=collect)
        torch.cuda.synchronize()
        a = st.out.clone()
        st.out.fill_(3.0)
        st.verify(collect=collect, host_plan=True)
        torch.cuda.synchronize()
        assert same_out(a, st.out), collect
        b = st.out.clone()
        st.verify(collect=collect, host_plan=True)     # host-planned calls are deterministic
        torch.cuda.synchronize()
        assert torch.equal(b.view(torch.uint8), st.out.view(torch.uint8)), collect
    if not isinstance(case, str):        # (the 128K-long ragged sequences have sampled checks of their own)
        st.run(fused=True, host_plan=True)
        torch.cuda.synchronize()
        check_layer(wl, inp, st)


@pytest.mark.parametrize("case", FUSED_CASES,
                         ids=lambda c: c if isinstance(c, str) else f"{c[0]}-B{c[1]}-{c[2]}x{c[3]}-D{c[4]}-g{c[5]}-L{c[6]}")
def test_verify_select_halves_on_two_streams_equal_one_call(case):
    """vegas_verify_select_begin_hostplan on one stream, then vegas_verify_select_end_hostplan on a
    second stream ordered after it by an event: output, scores and selection equal the one call's bit
    for bit, from any workspace contents, twice in a row."""
    if isinstance(case, str):
        wl = W.named_workload(4)
    else:
        dtype, B, hq, hkv, d, gamma, prefixes, ratio = case
        wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, ratio=ratio)
    log(f"case: verify+select halves on two streams {wl.name}")
    inp = W.make_inputs(wl, seed=6, device="cuda")
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts)
    cu, cuk = wl.cu_seqlens(), wl.cu_k()
    st.verify_select(host_plan=True)
    torch.cuda.synchronize()
    ref = (st.out.clone(), [st.scores[:, cu[b]:cu[b] + wl.prefix_lens[b]].clone() for b in range(wl.batch)],
           st.indices[: cuk[-1]].clone())
    side = torch.cuda.Stream()
    for rep, fill in enumerate((0x5A, 0xFF)):
        st.workspace.fill_(fill)
        st.out.fill_(3.0)
        st.scores.fill_(float("nan"))
        st.indices.fill_(-7)
        st.run(fused=True, host_plan=True, select_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(st.out.view(torch.uint8), ref[0].view(torch.uint8)), rep
        for b in range(wl.batch):
            assert torch.equal(st.scores[:, cu[b]:cu[b] + wl.prefix_lens[b]], ref[1][b]), (rep, b)
        assert torch.equal(st.indices[: cuk[-1]], ref[2]), rep
    if not isinstance(case, str):
        check_layer(wl, inp, st)
