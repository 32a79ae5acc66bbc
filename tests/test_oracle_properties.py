"""Property-based checks of the oracle on random small shapes (CPU only): head dims
D in {4, 8, 64}, GQA groups G in {1, 2, 4, 8}, gamma in 0..7, prefixes of 0..300 positions.
Each property follows from the definitions the oracle implements, not from the oracle's own
formulas: softmax rows are probability distributions; the result agrees with a library
attention (torch, float64) under the same mask; only rows 0 and gamma enter the collected
score ("Vegas ..." sec. 3.3); scaling s by 2 scales every logit exactly; sparse attention
over the whole visible range is full attention; the selected set maximises the summed score
over all k-subsets (summary sec. 2A), by brute force on short prefixes."""
import itertools

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=30, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def layer(draw, max_prefix=300):
    d = draw(st.sampled_from([4, 8, 64]))
    hkv = draw(st.sampled_from([1, 2]))
    G = draw(st.sampled_from([1, 2, 4, 8]))
    gamma = draw(st.integers(0, 7))
    batch = draw(st.integers(1, 3))
    prefixes = draw(st.lists(st.integers(0, max_prefix), min_size=batch, max_size=batch))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    W = gamma + 1
    lens = [p + W for p in prefixes]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((batch * W, hkv * G, d)).astype(np.float32)
    k = rng.standard_normal((total, hkv, d)).astype(np.float32)
    v = rng.standard_normal((total, hkv, d)).astype(np.float32)
    return dict(q=q, k=k, v=v, cu=cu, gamma=gamma, G=G, hkv=hkv, d=d, prefixes=prefixes,
                scale=float(d) ** -0.5, rng=rng)


def torch_reference(c):
    """float64 torch attention, row r of sequence b seeing keys 0 .. L_b + r."""
    W = c["gamma"] + 1
    outs = []
    for b, L in enumerate(c["prefixes"]):
        s0, s1 = c["cu"][b], c["cu"][b + 1]
        q = torch.from_numpy(c["q"][b * W:(b + 1) * W]).double().transpose(0, 1)       # [Hq, W, D]
        k = torch.from_numpy(c["k"][s0:s1]).double().repeat_interleave(c["G"], dim=1).transpose(0, 1)
        v = torch.from_numpy(c["v"][s0:s1]).double().repeat_interleave(c["G"], dim=1).transpose(0, 1)
        n = s1 - s0
        mask = torch.arange(n)[None, :] <= (L + torch.arange(W))[:, None]             # [W, n]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=c["scale"])
        outs.append(o.transpose(0, 1).numpy())
    return np.concatenate(outs)


@SETTINGS
@given(layer())
def test_rows_are_distributions_and_match_torch(c):
    ones = np.ones_like(c["v"])
    o1, _ = oracle.verify_attn(c["q"], c["k"], ones, c["cu"], c["gamma"], c["scale"], want_scores=False)
    assert np.allclose(o1, 1.0, rtol=0, atol=1e-12)               # weights sum to one
    o, _ = oracle.verify_attn(c["q"], c["k"], c["v"], c["cu"], c["gamma"], c["scale"], want_scores=False)
    assert np.allclose(o, torch_reference(c), rtol=0, atol=1e-10)


@SETTINGS
@given(layer())
def test_only_rows_zero_and_gamma_are_collected(c):
    _, s = oracle.verify_attn(c["q"], c["k"], c["v"], c["cu"], c["gamma"], c["scale"])
    q2 = c["q"].copy()
    W = c["gamma"] + 1
    for b in range(len(c["prefixes"])):
        for r in range(1, W - 1):                                   # rows strictly between 0 and gamma
            q2[b * W + r] = c["rng"].standard_normal(q2.shape[1:]).astype(np.float32)
    _, s2 = oracle.verify_attn(q2, c["k"], c["v"], c["cu"], c["gamma"], c["scale"])
    assert np.array_equal(s, s2)
    _, sd = oracle.verify_attn(c["q"], c["k"], c["v"], c["cu"], c["gamma"], 2 * c["scale"])
    for b, L in enumerate(c["prefixes"]):
        sl = slice(c["cu"][b], c["cu"][b] + L)
        assert np.array_equal(sd[:, sl], 2 * s[:, sl])             # a power-of-two scale is exact
        # the collected score is the logit sum written out over heads and the two rows
        if L:
            W0, Wg = b * W, b * W + c["gamma"]
            rows = {W0, Wg}
            ref = np.zeros((c["hkv"], L))
            for g in range(c["hkv"]):
                for h in range(g * c["G"], (g + 1) * c["G"]):
                    for r in rows:
                        ref[g] += c["scale"] * (c["k"][c["cu"][b]:c["cu"][b] + L, g].astype(np.float64)
                                                @ c["q"][r, h].astype(np.float64))
            assert np.allclose(s[:, sl], ref, rtol=1e-12, atol=1e-10)


@SETTINGS
@given(layer(max_prefix=60))
def test_sparse_over_the_visible_range_is_full_attention(c):
    o, _ = oracle.verify_attn(c["q"], c["k"], c["v"], c["cu"], c["gamma"], c["scale"], want_scores=False)
    W = c["gamma"] + 1
    r = int(c["rng"].integers(0, W))                               # one verification row per sequence
    qd = np.stack([c["q"][b * W + r] for b in range(len(c["prefixes"]))])
    lists = [np.arange(L + r + 1, dtype=np.int32) for L in c["prefixes"]]
    idx = np.concatenate(lists)
    cui = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    od = oracle.sparse_decode_attn(qd, c["k"], c["v"], c["cu"], idx, cui, c["scale"])
    for b in range(len(c["prefixes"])):
        assert np.allclose(od[b], o[b * W + r], rtol=0, atol=1e-12)


@SETTINGS
@given(st.integers(1, 10), st.integers(1, 3), st.integers(0, 2 ** 31 - 1), st.booleans())
def test_selection_maximises_the_summed_score(L, hkv, seed, ties):
    rng = np.random.default_rng(seed)
    gamma = 1
    n = L + gamma + 1
    cu = np.array([0, n], np.int32)
    s = rng.integers(-3, 4, size=(hkv, n)).astype(np.float64) if ties else rng.standard_normal((hkv, n))
    S = s.sum(axis=0)[:L]
    for k in range(0, L + 1):
        t, _, _ = oracle.select_topk(s, cu, gamma, np.array([0, k], np.int32))
        best = max((sum(S[list(c)]) for c in itertools.combinations(range(L), k)), default=0.0)
        assert len(t) == k and np.all(np.diff(t) > 0)
        assert sum(S[t]) == pytest.approx(best, abs=1e-12)
        # among equal maxima the lower positions are taken: the set is the lexicographically first
        first = next(c for c in itertools.combinations(range(L), k)
                     if abs(sum(S[list(c)]) - best) <= 1e-12) if k else ()
        if ties:
            assert tuple(t) == first
