"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here retypes the oracle's formulas: every check is a closed form, an
invariant, a brute force over sets, a hand-worked fixture, or an independent
library routine (torch's fp64 attention and topk).  A plausible mistake in the
oracle -- a dropped collected row, a wrong GQA head map, an off-by-one causal
mask, a wrong tie order -- fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, batch, hq, hkv, d, gamma, prefix_lens, dtype="f32"):
    rng = np.random.default_rng(seed)
    W = gamma + 1
    lens = [L + W for L in prefix_lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((batch * W, hq, d)).astype(np.float32)
    k = rng.standard_normal((total, hkv, d)).astype(np.float32)
    v = rng.standard_normal((total, hkv, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                   for x in (q, k, v))
    return q, k, v, cu


def as_f64(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------- golden fixtures

def test_golden_softmax_ln123():
    g = json.load(open(os.path.join(GOLDEN, "softmax_ln123.json")))
    s = g["softmax_scale"]
    q = np.zeros((1, 1, 4), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((3, 1, 4), np.float32)
    v = np.zeros((3, 1, 4), np.float32)
    for j in range(3):
        k[j, 0, 0] = math.log(j + 1) / s
        v[j, 0, j] = 1.0
    out, scores = oracle.verify_attn(q, k, v, [0, 3], gamma=0, scale=s)
    expect = [1 / 6, 1 / 3, 1 / 2, 0.0]
    assert np.allclose(out[0, 0], expect, atol=1e-6, rtol=0)
    # the two prefix positions carry their logits ln 1, ln 2 (row 0 is collected once)
    assert np.allclose(scores[0, :2], [0.0, math.log(2)], atol=1e-6)


def test_golden_topk_hand():
    g = json.load(open(os.path.join(GOLDEN, "topk_hand.json")))
    c = np.array(g["kv_head_scores"], dtype=np.float64)
    c = np.concatenate([c, np.full((2, 1), 100.0)], axis=1)   # one verification row: never a candidate
    L = c.shape[1] - 1
    for case in g["cases"]:
        idx, theta, S = oracle.select_topk(c, [0, L + 1], gamma=0, cu_k=[0, case["k"]])
        assert idx.tolist() == case["T"], case
        assert np.array_equal(S[:L], np.array(g["summed_score"], np.float64))


# ---------------------------------------------------------------- attention closed forms

@pytest.mark.parametrize("hq,hkv,gamma", [(4, 1, 3), (4, 4, 0), (8, 2, 5)])
def test_probabilities_sum_to_one(hq, hkv, gamma):
    """With one-hot value rows e_(j mod D) the output sums to the total softmax mass."""
    d = 16
    q, k, v, cu = rand_case(1, 2, hq, hkv, d, gamma, [37, 5])
    v[:] = 0
    for j in range(v.shape[0]):
        v[j, :, j % d] = 1.0
    out, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=0.3)
    assert np.abs(out.sum(-1) - 1.0).max() < 1e-12
    assert (out >= 0).all()


def test_zero_keys_give_mean_of_visible_values():
    gamma, L = 3, 20
    q, k, v, cu = rand_case(2, 1, 2, 1, 8, gamma, [L])
    k[:] = 0
    out, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=1.0)
    vd = v.astype(np.float64)
    for r in range(gamma + 1):
        mean = vd[: L + r + 1, 0].mean(axis=0)
        assert np.allclose(out[r, 0], mean, atol=1e-12, rtol=0)
        assert np.allclose(out[r, 1], mean, atol=1e-12, rtol=0)


def test_empty_prefix_first_row_sees_one_key():
    gamma = 2
    q, k, v, cu = rand_case(3, 1, 2, 2, 8, gamma, [0])
    out, scores = oracle.verify_attn(q, k, v, cu, gamma, scale=0.7)
    for h in range(2):
        assert np.array_equal(out[0, h], v[0, h].astype(np.float64))


def test_causal_mask_boundary():
    """Row r is unaffected by keys/values after position L+r and affected by position L+r."""
    gamma, L = 4, 9
    q, k, v, cu = rand_case(4, 1, 2, 1, 8, gamma, [L])
    base, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=0.5)
    for r in range(gamma + 1):
        k2, v2 = k.copy(), v.copy()
        k2[L + r + 1:] += 3.0
        v2[L + r + 1:] -= 5.0
        o2, _ = oracle.verify_attn(q, k2, v2, cu, gamma, scale=0.5)
        assert np.array_equal(o2[r], base[r])
        k3 = k.copy()
        k3[L + r] += 1.0
        o3, _ = oracle.verify_attn(q, k3, v, cu, gamma, scale=0.5)
        assert not np.allclose(o3[r], base[r], atol=1e-9)


def sdpa_reference(q, k, v, cu, gamma, scale, hq, hkv):
    """torch fp64 scaled_dot_product_attention with repeat-interleaved KV and an explicit
    bottom-right causal mask, sequence by sequence."""
    W = gamma + 1
    G = hq // hkv
    outs = []
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        L = n - W
        qb = torch.from_numpy(as_f64(q[b * W:(b + 1) * W])).permute(1, 0, 2)       # [Hq, W, D]
        kb = torch.from_numpy(as_f64(k[s0:s1])).permute(1, 0, 2).repeat_interleave(G, 0)
        vb = torch.from_numpy(as_f64(v[s0:s1])).permute(1, 0, 2).repeat_interleave(G, 0)
        mask = torch.arange(n)[None, :] <= (L + torch.arange(W))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=scale)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("batch,hq,hkv,d,gamma,prefix", [
    (1, 4, 1, 64, 3, [100]),
    (3, 8, 2, 32, 5, [50, 1, 77]),
    (2, 6, 3, 16, 0, [13, 40]),
])
def test_verify_matches_torch_sdpa(dtype, batch, hq, hkv, d, gamma, prefix):
    q, k, v, cu = rand_case(5, batch, hq, hkv, d, gamma, prefix, dtype)
    out, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=0.125)
    ref = sdpa_reference(q, k, v, cu, gamma, 0.125, hq, hkv)
    assert np.abs(out - ref).max() < 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    gamma, hq, hkv = 2, 8, 2
    q, k, v, cu = rand_case(6, 2, hq, hkv, 16, gamma, [30, 12])
    out_gqa, sc_gqa = oracle.verify_attn(q, k, v, cu, gamma, scale=0.25)
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    out_mha, sc_mha = oracle.verify_attn(q, kr, vr, cu, gamma, scale=0.25)
    assert np.abs(out_gqa - out_mha).max() < 1e-12
    # the per-KV-head score is the sum of the MHA per-head scores of its group
    sc_group = sc_mha.reshape(hkv, hq // hkv, -1).sum(axis=1)
    assert np.abs(sc_gqa - sc_group).max() < 1e-9


# ---------------------------------------------------------------- Collect-2-Query

def test_only_first_and_last_rows_are_collected():
    gamma, L = 5, 40
    q, k, v, cu = rand_case(7, 2, 4, 2, 16, gamma, [L, L])
    _, base = oracle.verify_attn(q, k, v, cu, gamma, scale=0.3)
    W = gamma + 1
    for r in range(W):
        q2 = q.copy()
        q2[r::W] += 0.5          # perturb row r of every sequence
        _, s2 = oracle.verify_attn(q2, k, v, cu, gamma, scale=0.3)
        prefix = np.concatenate([np.arange(cu[b], cu[b] + L) for b in range(2)])
        if r in (0, gamma):
            assert np.all(np.abs(s2[:, prefix] - base[:, prefix]) > 0)
        else:
            assert np.array_equal(s2, base)


def test_collected_score_with_one_hot_keys():
    """With key i = one-hot e_i the logit of (row r, head h) at position i is scale*q[r,h,i],
    so the collected score is scale * the sum of those query entries over rows {0, gamma}
    and over the heads of the KV group."""
    gamma, hq, hkv, d, L = 3, 6, 2, 32, 20
    q, k, v, cu = rand_case(8, 1, hq, hkv, d, gamma, [L])
    k[:] = 0
    for i in range(k.shape[0]):
        k[i, :, i] = 1.0
    s = 0.75
    _, scores = oracle.verify_attn(q, k, v, cu, gamma, scale=s)
    G = hq // hkv
    for g in range(hkv):
        for i in range(L):
            want = s * sum(float(q[r, h, i]) for r in (0, gamma) for h in range(g * G, (g + 1) * G))
            assert abs(scores[g, i] - want) < 1e-9
    assert np.all(scores[:, L:] == 0)     # verification rows are not candidates: untouched


def test_gamma_zero_collects_row_once():
    q, k, v, cu = rand_case(9, 1, 2, 1, 8, 0, [10])
    _, s_set = oracle.verify_attn(q, k, v, cu, 0, scale=1.0)             # mask {0} | {0}
    _, s_all = oracle.verify_attn(q, k, v, cu, 0, scale=1.0, collect_mask=1)
    assert np.array_equal(s_set, s_all)


# ---------------------------------------------------------------- selection

def test_topk_brute_force_over_sets():
    rng = np.random.default_rng(10)
    for trial in range(40):
        L = int(rng.integers(1, 11))
        hkv = int(rng.integers(1, 4))
        kb = int(rng.integers(0, L + 1))
        c = rng.standard_normal((hkv, L + 1))
        if trial % 4 == 0:
            c = np.round(c * 2) / 2          # force ties
        idx, theta, _ = oracle.select_topk(c, [0, L + 1], 0, [0, kb])
        best = -np.inf
        best_sets = []
        for T in itertools.combinations(range(L), kb):
            obj = sum(c[g, list(T)].sum() for g in range(hkv)) if kb else 0.0
            if obj > best + 1e-12:
                best, best_sets = obj, [T]
            elif abs(obj - best) <= 1e-12:
                best_sets.append(T)
        got = sum(c[g, idx].sum() for g in range(hkv)) if kb else 0.0
        assert abs(got - best) <= 1e-9
        assert tuple(idx.tolist()) in best_sets
        # among the optimal sets, the lexicographically smallest (lower positions win ties)
        assert tuple(idx.tolist()) == min(best_sets)


def test_topk_matches_torch_topk_on_distinct_scores():
    rng = np.random.default_rng(11)
    L, W = 5000, 4
    cu = [0, L + W, 2 * (L + W)]
    c = rng.standard_normal((3, cu[-1]))
    kb = 321
    idx, theta, S = oracle.select_topk(c, cu, W - 1, [0, kb, 2 * kb])
    for b in range(2):
        Sb = torch.from_numpy(c[:, cu[b]:cu[b] + L]).sum(0)
        vals, pos = torch.topk(Sb, kb)
        assert idx[b * kb:(b + 1) * kb].tolist() == sorted(pos.tolist())
        assert theta[b] == pytest.approx(float(vals[-1]), abs=1e-12)


def test_all_ties_take_lowest_positions():
    """Q = 0 makes every logit 0, so every prefix score ties and T = [0, k)."""
    gamma, L = 2, 64
    q, k, v, cu = rand_case(12, 2, 4, 2, 16, gamma, [L, L])
    q[:] = 0
    _, scores = oracle.verify_attn(q, k, v, cu, gamma, scale=1.0)
    idx, _, _ = oracle.select_topk(scores, cu, gamma, [0, 5, 5 + 17])
    assert idx.tolist() == list(range(5)) + list(range(17))


def test_topk_edge_sizes_and_scale_invariance():
    rng = np.random.default_rng(13)
    L, gamma = 50, 1
    cu = [0, L + 2]
    c = rng.standard_normal((2, L + 2))
    e, _, _ = oracle.select_topk(c, cu, gamma, [0, 0])
    assert e.size == 0
    a, _, _ = oracle.select_topk(c, cu, gamma, [0, L])
    assert a.tolist() == list(range(L))
    t1, _, _ = oracle.select_topk(c, cu, gamma, [0, 9])
    t2, _, _ = oracle.select_topk(c * 3.5, cu, gamma, [0, 9])
    assert t1.tolist() == t2.tolist()
    with pytest.raises(ValueError):
        oracle.select_topk(c, cu, gamma, [0, L + 1])


# ---------------------------------------------------------------- sparse decode

def test_sparse_full_prefix_equals_verification_row():
    """Sparse attention whose list is every key row r sees equals verification row r."""
    gamma, hq, hkv, d = 3, 4, 2, 16
    prefix = [25, 7]
    q, k, v, cu = rand_case(14, 2, hq, hkv, d, gamma, prefix)
    out, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=0.4)
    W = gamma + 1
    for r in range(W):
        qd = np.stack([q[b * W + r] for b in range(2)])
        lists = [np.arange(prefix[b] + r + 1, dtype=np.int32) for b in range(2)]
        cui = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
        od = oracle.sparse_decode_attn(qd, k, v, cu, np.concatenate(lists), cui, scale=0.4)
        for b in range(2):
            assert np.abs(od[b] - out[b * W + r]).max() < 1e-12


def test_sparse_single_index_and_empty_list():
    q, k, v, cu = rand_case(15, 2, 4, 2, 8, 1, [10, 10])
    qd = q[:2]
    od = oracle.sparse_decode_attn(qd, k, v, cu, np.array([6], np.int32), [0, 1, 1], scale=1.0)
    for h in range(4):
        assert np.array_equal(od[0, h], v[cu[0] + 6, h // 2].astype(np.float64))
    assert np.all(od[1] == 0)


def test_sparse_list_order_irrelevant_and_matches_sdpa():
    rng = np.random.default_rng(16)
    q, k, v, cu = rand_case(16, 1, 8, 2, 32, 2, [200])
    qd = q[:1]
    lst = np.sort(rng.choice(203, 40, replace=False)).astype(np.int32)
    o1 = oracle.sparse_decode_attn(qd, k, v, cu, lst, [0, 40], scale=0.2)
    o2 = oracle.sparse_decode_attn(qd, k, v, cu, lst[::-1].copy(), [0, 40], scale=0.2)
    assert np.abs(o1 - o2).max() < 1e-13
    qb = torch.from_numpy(as_f64(qd[0]))[:, None, :]                                   # [Hq,1,D]
    kb = torch.from_numpy(as_f64(k[lst])).permute(1, 0, 2).repeat_interleave(4, 0)
    vb = torch.from_numpy(as_f64(v[lst])).permute(1, 0, 2).repeat_interleave(4, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, scale=0.2)[:, 0].numpy()
    assert np.abs(o1[0] - ref).max() < 1e-12


def test_oracle_rejects_bad_arguments():
    q, k, v, cu = rand_case(17, 1, 4, 2, 8, 1, [10])
    with pytest.raises(ValueError):
        oracle.sparse_decode_attn(q[:1], k, v, cu, np.array([12], np.int32), [0, 1], scale=1.0)
    with pytest.raises(ValueError):
        oracle.verify_attn(q, k, v, [0, 1], 1, scale=1.0)    # sequence shorter than gamma+1


# ---------------------------------------------------------------- local mask and StreamingLLM lists

def band_sdpa_reference(q, k, v, cu, gamma, scale, hq, hkv, window):
    """torch fp64 SDPA with an explicit band mask: row r sees L+r-window < j <= L+r."""
    W = gamma + 1
    G = hq // hkv
    outs = []
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        L = n - W
        qb = torch.from_numpy(as_f64(q[b * W:(b + 1) * W])).permute(1, 0, 2)
        kb = torch.from_numpy(as_f64(k[s0:s1])).permute(1, 0, 2).repeat_interleave(G, 0)
        vb = torch.from_numpy(as_f64(v[s0:s1])).permute(1, 0, 2).repeat_interleave(G, 0)
        j = torch.arange(n)[None, :]
        last = (L + torch.arange(W))[:, None]
        mask = (j <= last) & (j > last - window)
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=scale)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("window", [1, 3, 17, 128])
def test_local_mask_matches_torch_band_sdpa(window):
    gamma, hq, hkv, d = 3, 8, 2, 32
    q, k, v, cu = rand_case(18, 3, hq, hkv, d, gamma, [200, 5, 60], "bf16")
    out, sc = oracle.verify_attn(q, k, v, cu, gamma, scale=0.2, want_scores=False, window=window)
    assert sc is None
    ref = band_sdpa_reference(q, k, v, cu, gamma, 0.2, hq, hkv, window)
    assert np.abs(out - ref).max() < 1e-12


def test_window_one_sees_only_its_own_key():
    gamma = 4
    q, k, v, cu = rand_case(19, 2, 4, 2, 16, gamma, [30, 0])
    out, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=1.0, want_scores=False, window=1)
    W = gamma + 1
    for b in range(2):
        L = int(cu[b + 1] - cu[b]) - W
        for r in range(W):
            for h in range(4):
                assert np.array_equal(out[b * W + r, h], v[cu[b] + L + r, h // 2].astype(np.float64))


def test_local_mask_boundary():
    """Keys before the band do not matter; the first key inside it does."""
    gamma, L, window = 2, 50, 8
    q, k, v, cu = rand_case(20, 1, 2, 1, 8, gamma, [L])
    base, _ = oracle.verify_attn(q, k, v, cu, gamma, scale=0.5, want_scores=False, window=window)
    for r in range(gamma + 1):
        lo = L + r - window + 1
        k2, v2 = k.copy(), v.copy()
        k2[:lo] += 3.0
        v2[:lo] -= 2.0
        o2, _ = oracle.verify_attn(q, k2, v2, cu, gamma, scale=0.5, want_scores=False, window=window)
        assert np.array_equal(o2[r], base[r])
        k3 = k.copy()
        k3[lo] += 1.0
        o3, _ = oracle.verify_attn(q, k3, v, cu, gamma, scale=0.5, want_scores=False, window=window)
        assert not np.allclose(o3[r], base[r], atol=1e-9)


def test_local_mask_rejects_collection():
    q, k, v, cu = rand_case(21, 1, 2, 1, 8, 1, [20])
    with pytest.raises(ValueError):
        oracle.verify_attn(q, k, v, cu, 1, scale=1.0, window=4)


def test_streaming_lists_closed_form():
    gamma = 2
    lens = [100 + 3, 10 + 3, 7 + 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    budgets = [12, 10, 0]
    cui = np.concatenate([[0], np.cumsum(budgets)]).astype(np.int32)
    got = oracle.streaming_indices(cu, gamma, 4, cui)
    assert got[:12].tolist() == [0, 1, 2, 3] + list(range(92, 100))
    assert got[12:22].tolist() == list(range(10))          # budget = whole prefix
    got = oracle.streaming_indices(cu, gamma, 0, cui)
    assert got[:12].tolist() == list(range(88, 100))       # no sinks: pure sliding window
    with pytest.raises(ValueError):
        oracle.streaming_indices(cu, gamma, 4, np.array([0, 101, 101, 101], np.int32))


# ---------------------------------------------------------------- speculative-sampling acceptance

def _softmax_rows(rng, shape, temp=1.0):
    x = rng.standard_normal(shape) / temp
    e = np.exp(x - x.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def test_accept_greedy_special_case():
    """One-hot p and q (greedy decoding): a draft is kept iff it is the target's argmax, and the
    replacement at the first mismatch is the target's argmax."""
    rng = np.random.default_rng(30)
    B, gamma, V = 64, 4, 11
    g = rng.integers(0, V, (B, gamma + 1))
    drafts = np.where(rng.random((B, gamma)) < 0.7, g[:, :gamma], rng.integers(0, V, (B, gamma))).astype(np.int32)
    p = np.zeros((B, gamma + 1, V), np.float32)
    q = np.zeros((B, gamma, V), np.float32)
    for b in range(B):
        p[b, np.arange(gamma + 1), g[b]] = 1.0
        q[b, np.arange(gamma), drafts[b]] = 1.0
    n, t = oracle.spec_accept(p, q, drafts, rng.random((B, gamma)).astype(np.float32),
                              rng.random(B).astype(np.float32))
    for b in range(B):
        want = 0
        while want < gamma and drafts[b, want] == g[b, want]:
            want += 1
        assert n[b] == want
        assert t[b] == g[b, want]


def test_accept_identical_distributions_keep_every_draft():
    rng = np.random.default_rng(31)
    B, gamma, V = 16, 3, 50
    p = _softmax_rows(rng, (B, gamma + 1, V))
    q = p[:, :gamma].copy()
    drafts = rng.integers(0, V, (B, gamma)).astype(np.int32)
    n, _ = oracle.spec_accept(p, q, drafts, (rng.random((B, gamma)) * 0.999).astype(np.float32),
                              rng.random(B).astype(np.float32))
    assert np.all(n == gamma)


def test_draw_is_the_inverse_cdf_with_half_open_bins():
    p = np.array([[[0.25, 0.5, 0.25]]], np.float32)
    cases = {0.0: 0, 0.2499: 0, 0.25: 1, 0.7499: 1, 0.75: 2, 0.9999: 2}
    for u, want in cases.items():
        _, t = oracle.spec_accept(p, np.zeros((1, 0, 3), np.float32), np.zeros((1, 0), np.int32),
                                  np.zeros((1, 0), np.float32), np.array([u], np.float32))
        assert t[0] == want, (u, t[0], want)


def test_first_token_follows_the_target_distribution():
    """The lossless property: with y ~ q, the first emitted token (the kept draft, or the residual
    replacement) is distributed as p.  Integrate exactly over y and over grids of both uniforms."""
    rng = np.random.default_rng(32)
    V, N1, N2 = 5, 160, 160
    p1 = _softmax_rows(rng, (V,), 0.7)
    q1 = _softmax_rows(rng, (V,), 0.7)
    u1 = (np.arange(N1) + 0.5) / N1
    u2 = (np.arange(N2) + 0.5) / N2
    yy, a, s = np.meshgrid(np.arange(V), u1, u2, indexing="ij")
    B = yy.size
    p = np.broadcast_to(np.stack([p1, p1]), (B, 2, V)).copy()       # gamma = 1; p_2 unused unless kept
    q = np.broadcast_to(q1, (B, 1, V)).copy()
    n, t = oracle.spec_accept(p, q, yy.reshape(B, 1).astype(np.int32), a.reshape(B, 1).astype(np.float32),
                              s.reshape(B).astype(np.float32))
    first = np.where(n == 1, yy.reshape(B), t)
    w = q1[yy.reshape(B)] / (N1 * N2)                                 # probability weight of each instance
    emp = np.array([w[first == y].sum() for y in range(V)])
    assert np.abs(emp - p1).max() < 0.02
    # the acceptance rate is 1 - TV(p, q)
    assert abs(float(w[n == 1].sum()) - (1 - 0.5 * np.abs(p1 - q1).sum())) < 0.02


def test_all_kept_bonus_follows_the_last_target_row():
    rng = np.random.default_rng(33)
    V, N = 6, 4000
    p = _softmax_rows(rng, (1, 3, V))
    p = np.repeat(p, N, axis=0)
    q = p[:, :2].copy()
    drafts = np.zeros((N, 2), np.int32)
    n, t = oracle.spec_accept(p, q, drafts, np.zeros((N, 2), np.float32),
                              ((np.arange(N) + 0.5) / N).astype(np.float32))
    assert np.all(n == 2)
    emp = np.bincount(t, minlength=V) / N
    assert np.abs(emp - p[0, 2]).max() < 2.0 / N + 1e-6
