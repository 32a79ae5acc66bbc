"""Shared helpers of the GPU parity tests: run one layer step through the C ABI
and compare it with the CPU oracle on the same bits, by the rules:
  attention outputs   max |gpu - oracle| <= 2e-2 (bf16) or 1e-4 (fp32)
  collected scores    |gpu - oracle| <= 1e-3 * max(1, |oracle|)
  selection           exactly k_b unique ascending prefix positions; any
                      position where the GPU and oracle sets differ has an
                      oracle score within 1e-3 of the oracle's k-th largest
  drafting            the oracle is run on the GPU's own selected lists
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle
from verification_guided_sparse_verify_amd import workloads as W
from verification_guided_sparse_verify_amd.step import LayerStep

ATOL = {"bf16": 2e-2, "f32": 1e-4}
SCORE_RTOL = 1e-3
THETA_TOL = 1e-3


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MARGINS = os.path.join(ROOT, "gpurun_out", "parity_margins.json")


def record_margins(case: str, wl: W.Workload, worst: dict, seqs):
    """Keep a case's worst errors next to its tolerances in gpurun_out/parity_margins.json (one
    entry per case, merged with the entries of earlier cases), so the distance to each bound is
    on record, not only the pass."""
    atol = ATOL[wl.dtype]
    entry = {"workload": wl.name, "sequences_checked": list(seqs), "of": wl.batch,
             "out_max_abs_err": worst["out"], "out_tol": atol,
             "score_max_rel_err": worst["score"], "score_tol": SCORE_RTOL,
             "draft_max_abs_err": worst["draft"], "draft_tol": atol,
             "selection_diffs_outside_tie_band": 0,
             "selection_diffs_inside_tie_band": worst.get("sel_diff", 0)}
    os.makedirs(os.path.dirname(MARGINS), exist_ok=True)
    data = {}
    if os.path.exists(MARGINS):
        try:
            with open(MARGINS) as f:
                data = json.load(f)
        except (OSError, ValueError):
            data = {}
    data[case] = entry
    with open(MARGINS, "w") as f:
        json.dump(data, f, indent=1)
    log(f"  margins {case}: {json.dumps(entry)}")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_layer(wl: W.Workload, seed: int = 0, layer: int = 0, inputs=None, collect_mask=None):
    inp = inputs if inputs is not None else W.make_inputs(wl, seed=seed, device="cuda", layer=layer)
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts, collect_mask=collect_mask)
    st.run()
    torch.cuda.synchronize()
    return inp, st


def _seq_host(inp, wl: W.Workload, b: int):
    cu = wl.cu_seqlens()
    Wr = wl.gamma + 1
    s0, s1 = cu[b], cu[b + 1]
    q = W.host_bits(inp["q"][b * Wr:(b + 1) * Wr])
    k = W.host_bits(inp["k"][s0:s1])
    v = W.host_bits(inp["v"][s0:s1])
    return q, k, v, np.array([0, s1 - s0], np.int32)


def check_layer(wl: W.Workload, inp, st: LayerStep, seqs=None, check_drafts: bool = True,
                collect_mask=None):
    """Compare every listed sequence (default: all) with the oracle."""
    seqs = range(wl.batch) if seqs is None else seqs
    atol = ATOL[wl.dtype]
    cu = wl.cu_seqlens()
    cuk = wl.cu_k()
    Wr = wl.gamma + 1
    out_all = st.out.float()
    sc_all = st.scores
    idx_all = st.indices
    worst = {"out": 0.0, "score": 0.0, "draft": 0.0, "sel_diff": 0}
    for b in seqs:
        L = wl.prefix_lens[b]
        kb = wl.k_per_seq[b]
        q, k, v, cu1 = _seq_host(inp, wl, b)
        o_ref, s_ref = oracle.verify_attn(q, k, v, cu1, wl.gamma, wl.scale, collect_mask=collect_mask)
        o_gpu = out_all[b * Wr:(b + 1) * Wr].cpu().numpy()
        err = float(np.abs(o_gpu - o_ref).max())
        worst["out"] = max(worst["out"], err)
        assert err <= atol, f"seq {b}: verify out max abs err {err} > {atol}"
        s_gpu = sc_all[:, cu[b]:cu[b] + L].cpu().numpy().astype(np.float64)
        rel = np.abs(s_gpu - s_ref[:, :L]) / np.maximum(1.0, np.abs(s_ref[:, :L]))
        r = float(rel.max()) if L else 0.0
        worst["score"] = max(worst["score"], r)
        assert r <= SCORE_RTOL, f"seq {b}: collected score rel err {r}"
        # selection
        t_ref, theta, S = oracle.select_topk(s_ref, cu1, wl.gamma, np.array([0, kb], np.int32))
        t_gpu = idx_all[cuk[b]:cuk[b + 1]].cpu().numpy()
        assert t_gpu.shape[0] == kb
        if kb:
            assert np.all(np.diff(t_gpu) > 0), f"seq {b}: indices not strictly ascending"
            assert t_gpu[0] >= 0 and t_gpu[-1] < L, f"seq {b}: index outside the prefix"
        diff = set(t_gpu.tolist()) ^ set(t_ref.tolist())
        worst["sel_diff"] += len(diff)
        bad = [i for i in diff if abs(S[i] - theta[0]) > THETA_TOL]
        assert not bad, f"seq {b}: selection differs beyond the threshold band at {bad[:10]}"
        # drafting over the GPU's own list
        if check_drafts:
            for j in range(wl.n_drafts):
                dq = W.host_bits(inp["draft_q"][j][b:b + 1])
                d_ref = oracle.sparse_decode_attn(dq, k, v, cu1, t_gpu, np.array([0, kb], np.int32), wl.scale)
                d_gpu = st.draft_out[j][b:b + 1].float().cpu().numpy()
                e = float(np.abs(d_gpu - d_ref).max())
                worst["draft"] = max(worst["draft"], e)
                assert e <= atol, f"seq {b} draft {j}: max abs err {e} > {atol}"
    return worst
