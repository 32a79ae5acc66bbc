"""Benchmark of the Vegas attention hot path on one MI355X.

One step is one speculative decode iteration of the 128K Qwen3-8B-shaped
workload (batch 4, 36 layers each with its own KV cache, 32 query / 8 KV
heads, head_dim 128, prefix 131072, gamma 5, k = 5% = 6553 per sequence and
layer, bf16): the verification pass runs verify (with Collect-2-Query) and
select on every layer, then gamma drafting passes run the sparse decode on
every layer.  The reported value is microseconds per layer-step
(verify + select + gamma drafts of one layer) = step time / layers.

With several layers, verification + selection runs as the one call in two
halves: the selections (keys, candidates, write) of a group of nine layers go
to a second stream after the group's last verification, beside the next
layers' verifications (the selected positions are used only by the drafting
passes, which wait for each group's selections).

Each step of several layers ends with a synchronisation, as a decoding loop's
iteration does: the next iteration's host-planned calls take host copies of
sequence lengths that depend on the tokens this iteration accepts.

Inputs are seeded synthetic tensors resident in HBM before timing starts.
The timed region runs the steps with no timing events (an event around every
call adds ~7 us per layer-step).  Further steps after it, with HIP events on
the launch stream around every call, give the per-call durations: those of
the verification calls (the dominant kernel) and the algorithmic bytes of one
call (each KV byte of the verified cache read once, Q and O, the collected
scores written once) give the HBM roofline figure.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure
METRIC = "µs per layer-step (verify+select+gamma drafts) and achieved HBM GB/s vs peak"


def algorithmic_bytes(wl):
    """Bytes the method must move, per call type, for one layer."""
    es = 2 if wl.dtype == "bf16" else 4
    B, Hq, Hkv, D, Wr = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma + 1
    total_kv = wl.total_kv
    sumL = sum(wl.prefix_lens)
    sumk = sum(wl.k_per_seq)
    kv = total_kv * Hkv * D * es * 2
    qo = B * Wr * Hq * D * es * 2
    scores = Hkv * sumL * 4
    verify = kv + qo + scores
    select = scores + sumk * 4
    draft = sumk * Hkv * D * es * 2 + sumk * 4 + B * Hq * D * es * 2
    return {"verify": verify, "select": select, "draft": draft,
            "layer_step": verify + select + wl.n_drafts * draft}


def product_code_lines(text):
    """The lines of a kernel source that the product build compiles, without comments, blank
    lines and the measurement-only VEGAS_PHASE_TRACE branches (their #else branches stay)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    state = ""                         # "trace": inside the trace branch; "else": in its #else branch
    out = []
    for ln in text.splitlines():
        code = re.sub(r"//.*", "", ln).strip()
        if code == "#ifdef VEGAS_PHASE_TRACE":
            state = "trace"
            continue
        if state and code == "#else":
            state = "else"
            continue
        if state and code == "#endif":
            state = ""
            continue
        if code and state != "trace":
            out.append(code)
    return out


def kernel_source_hash():
    """Hash of the attention kernels' product code (product_code_lines): a change of comments or
    of the trace build alone leaves the product kernels, and so the counters, as they were."""
    h = hashlib.sha256()
    for f in ("attn.hip", "internal.h", "select_device.h"):
        with open(os.path.join(ROOT, "verification_guided_sparse_verify_amd", "csrc", f)) as fh:
            for code in product_code_lines(fh.read()):
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(profile_name, launches_key):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, _, v = ln.partition("=")
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv[launches_key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, layer_inputs, min_seconds=10.0):
    """Time the CPU oracle on whole layers of the same workload (verify, select over the
    oracle's own scores, gamma drafts over the oracle's own selection), one layer after
    another until at least `min_seconds` of CPU work, and scale to one layer-step."""
    import numpy as np
    import oracle
    from verification_guided_sparse_verify_amd import workloads as W

    cus = np.array(wl.cu_seqlens(), np.int32)
    cuk = np.array(wl.cu_k(), np.int32)
    oracle._lib()
    spent, done, per_layer = 0.0, 0, []
    for inp in layer_inputs:
        q = W.host_bits(inp["q"])
        k = W.host_bits(inp["k"])
        v = W.host_bits(inp["v"])
        dq = W.host_bits(inp["draft_q"])
        t0 = time.perf_counter()
        _, sc = oracle.verify_attn(q, k, v, cus, wl.gamma, wl.scale)
        idx, _, _ = oracle.select_topk(sc, cus, wl.gamma, cuk)
        for j in range(wl.n_drafts):
            oracle.sparse_decode_attn(dq[j], k, v, cus, idx, cuk, wl.scale)
        dt = time.perf_counter() - t0
        spent += dt
        per_layer.append(dt)
        done += 1
        del q, k, v, dq, sc
        if spent >= min_seconds and done >= 3:
            break
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = int(omp) if omp and omp.isdigit() else len(os.sched_getaffinity(0))
    tasks = wl.batch * wl.num_kv_heads
    return {
        "value": round(spent * 1e6 / done, 1),
        "unit": "us/layer-step",
        "median_us": round(statistics.median(per_layer) * 1e6, 1),
        "per_layer_us": [round(x * 1e6, 1) for x in per_layer],
        "cores": min(threads, tasks),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"layers 0..{done - 1} of {len(layer_inputs)}, all {wl.batch} sequences "
                   f"(verify + select + {wl.n_drafts} drafts each), {spent:.2f} s in total, "
                   f"divided by {done} layer-steps (at least 3 layers; median_us is their median)"),
    }


def tiny_single_thread_oracle(repeats=3):
    """The oracle on one host thread for the tiny fp32 MQA configuration (1 sequence, 1024 positions,
    gamma 3): median of `repeats` whole layer-steps (verify + select + 3 drafts) after one warm-up."""
    import ctypes
    import numpy as np
    import oracle
    from verification_guided_sparse_verify_amd import workloads as W

    gomp = ctypes.CDLL("libgomp.so.1")          # the oracle's OpenMP runtime (gcc -fopenmp)
    prev = gomp.omp_get_max_threads()
    gomp.omp_set_num_threads(1)
    try:
        wl = W.named_workload(0)
        inp = W.make_inputs(wl, seed=0, device="cpu")
        q, k, v, dq = (W.host_bits(inp[n]) for n in ("q", "k", "v", "draft_q"))
        cus = np.array(wl.cu_seqlens(), np.int32)
        cuk = np.array(wl.cu_k(), np.int32)
        times = []
        for _ in range(repeats + 1):
            t0 = time.perf_counter()
            _, sc = oracle.verify_attn(q, k, v, cus, wl.gamma, wl.scale)
            idx, _, _ = oracle.select_topk(sc, cus, wl.gamma, cuk)
            for j in range(wl.n_drafts):
                oracle.sparse_decode_attn(dq[j], k, v, cus, idx, cuk, wl.scale)
            times.append(time.perf_counter() - t0)
    finally:
        gomp.omp_set_num_threads(prev)
    return {"workload": wl.name, "value": round(statistics.median(times[1:]) * 1e6, 1), "unit": "us/layer-step",
            "cores": 1, "kind": "oracle", "sample": f"median of {repeats} layer-steps after one warm-up"}


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_read_ceiling(nbytes: int = 4 << 30, reps: int = 5):
    """Best HBM streaming-read rate of a plain read kernel (libvegas_probe.so) over a few
    workgroup counts: a measured practical peak next to the published one.  The probe reads
    with the attention kernels' own load path (direct-to-LDS, non-temporal policy), the
    fastest of the read paths tried on MI355X."""
    import ctypes
    import torch
    from verification_guided_sparse_verify_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    probe = ctypes.CDLL(B.PROBE_LIB)
    fn = probe.vegas_probe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = (0.0, 0)
    for wgs in (256, 512, 1024, 2048, 4096):
        times = []
        for r in range(reps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = fn(buf.data_ptr(), nbytes, wgs, sink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"vegas_probe_stream_read returned {rc}")
            times.append((a, b))
        torch.cuda.synchronize()
        us = min(x.elapsed_time(y) for x, y in times[1:]) * 1e3
        gbps = nbytes / (us * 1e-6) / 1e9
        if gbps > best[0]:
            best = (gbps, wgs)
    del buf, sink
    return {"gbps": round(best[0], 1), "workgroups": best[1], "bytes": nbytes,
            "kernel": "vegas_probe_stream_read (16-byte non-temporal direct-to-LDS copies, 8 KB in flight per wave)"}


def gather_read_ceiling(wl, layer_inputs, steps, reps=3):
    """Best HBM rate of a plain gather kernel (libvegas_probe.so) reading exactly the bytes of the
    drafting passes: the K and V slices of every KV head of the selected rows of every layer (rows
    cold, layer after layer, as in the timed steps), over a few workgroup counts and depths of
    blocks in flight.  A measured practical peak for the drafting call, next to the published one."""
    import ctypes
    import torch
    from verification_guided_sparse_verify_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    probe = ctypes.CDLL(B.PROBE_LIB)
    fn = probe.vegas_probe_gather_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    es = 2 if wl.dtype == "bf16" else 4
    slice_bytes = wl.head_dim * es
    row_bytes = wl.num_kv_heads * slice_bytes
    cu, cuk = wl.cu_seqlens(), wl.cu_k()
    offs = torch.repeat_interleave(torch.tensor(cu[:-1], dtype=torch.int32),
                                   torch.tensor(wl.k_per_seq)).to("cuda")
    lists = [(inp["k"], inp["v"], (st.indices[: cuk[-1]] + offs).contiguous()) for inp, st in zip(layer_inputs, steps)]
    nbytes = sum(int(r.numel()) for _, _, r in lists) * row_bytes * 2
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = (0.0, 0, 0, 0)
    for hpw in ((1, 2) if wl.num_kv_heads % 2 == 0 else (1,)):
        for wgs in (256, 512, 1024):
            for inflight in (1, 2, 3):
                times = []
                for r in range(reps + 1):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for k, v, rows in lists:
                        rc = fn(k.data_ptr(), v.data_ptr(), rows.data_ptr(), rows.numel(), wl.total_kv, row_bytes,
                                slice_bytes, wl.num_kv_heads, hpw, wgs, inflight, sink.data_ptr(),
                                stream.cuda_stream)
                        if rc != 0:
                            raise RuntimeError(f"vegas_probe_gather_read returned {rc}")
                    b.record(stream)
                    times.append((a, b))
                torch.cuda.synchronize()
                us = min(x.elapsed_time(y) for x, y in times[1:]) * 1e3
                gbps = nbytes / (us * 1e-6) / 1e9
                if gbps > best[0]:
                    best = (gbps, wgs, inflight, hpw)
    return {"gbps": round(best[0], 1), "workgroups": best[1], "blocks_in_flight_per_wave": best[2],
            "heads_per_workgroup": best[3], "bytes": nbytes, "layers": len(lists),
            "kernel": ("vegas_probe_gather_read (the drafting pass's K/V slices of the selected rows of every "
                       "layer, 16-byte non-temporal direct-to-LDS copies, no arithmetic; best of 1 or 2 heads per "
                       "workgroup, 256-1024 workgroups and 1-3 blocks in flight per wave)")}


def launch_floor(chain: int = 200, reps: int = 5):
    """Cost of one kernel boundary in a chain of dependent launches on one stream
    (libvegas_probe.so's empty chained kernel), for one workgroup and for one round of 256
    workgroups holding 64 KB of LDS each (one per CU, as the attention kernels run): the floor
    under each small dependent kernel of a pass.  The chain is queued behind a 5 ms wait on the
    GPU, so it is timed at the GPU's rate rather than the host's launch rate."""
    import ctypes
    import torch
    from verification_guided_sparse_verify_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    probe = ctypes.CDLL(B.PROBE_LIB)
    fn = probe.vegas_probe_launch_chain
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    delay = probe.vegas_probe_delay
    delay.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    delay.restype = ctypes.c_int
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for name, wgs, lds in (("one_workgroup", 1, 0), ("256_workgroups_64kb_lds", 256, 65536)):
        times = []
        for r in range(reps + 1):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            # hold the GPU for 5 ms while the host queues the chain: the chain is then timed on
            # the GPU alone, not at the host's launch rate
            if delay(500000, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("vegas_probe_delay failed")
            a.record(stream)
            rc = fn(chain, wgs, lds, sink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"vegas_probe_launch_chain returned {rc}")
            times.append((a, b))
        torch.cuda.synchronize()
        out[name] = round(statistics.median(x.elapsed_time(y) for x, y in times[1:]) * 1e3 / chain, 2)
    out["unit"] = "us per dependent launch"
    out["kernel"] = (f"vegas_probe_launch_chain ({chain} chained launches of an empty kernel queued behind "
                     f"vegas_probe_delay, median of {reps})")
    return out


def collect_sweep(base, gammas=(1, 3, 5, 7, 11, 15), reps=8):
    """Verification time of one layer of `base` (its prefix, heads and batch) with collection
    off, Collect-2-Query (rows 0 and gamma) and all gamma+1 rows, for several gamma.  The pages
    report that collecting every row of an instrumented FlashAttention-3 grows with the row
    count while Collect-2-Query stays flat ("Vegas ...", sec. 3.3, Fig. 6); here collection is
    a head-summed reduction inside the kernel, whose cost does not depend on which rows are
    collected.  Prints one JSON line."""
    import dataclasses
    import torch
    from verification_guided_sparse_verify_amd import workloads as W
    from verification_guided_sparse_verify_amd.step import LayerStep

    stream = torch.cuda.current_stream()
    rows = []
    for gamma in gammas:
        if (gamma + 1) * (base.num_q_heads // base.num_kv_heads) > 64:
            continue
        wl = dataclasses.replace(base, gamma=gamma, layers=1, draft_steps=1)
        inps = [W.make_inputs(wl, seed=0, device="cuda:0", layer=l) for l in range(2)]
        masks = {"off": 0, "collect2": 1 | (1 << gamma), "all_rows": (1 << (gamma + 1)) - 1}
        res = {"gamma": gamma, "query_rows_per_kv_head": (gamma + 1) * (wl.num_q_heads // wl.num_kv_heads)}
        for name, mask in masks.items():
            steps = [LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, gamma, wl.seqlens,
                               wl.k_per_seq, wl.scale, n_drafts=1, collect_mask=mask if mask else None)
                     for inp in inps]
            calls = [st.bind(stream)[0 if mask else 1] for st in steps]
            for c in calls:
                c()
            pairs = []
            for _ in range(reps):
                for c in calls:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    c()
                    b.record(stream)
                    pairs.append((a, b))
            torch.cuda.synchronize()
            res[name + "_us"] = round(statistics.fmean(a.elapsed_time(b) * 1e3 for a, b in pairs), 2)
            del steps, calls
        res["collect2_overhead"] = round(res["collect2_us"] / res["off_us"] - 1, 4)
        res["all_rows_overhead"] = round(res["all_rows_us"] / res["off_us"] - 1, 4)
        rows.append(res)
        print(f"# gamma {gamma}: {res}", file=sys.stderr, flush=True)
        del inps
        torch.cuda.empty_cache()
    print(json.dumps({"collect_sweep": base.name, "unit": "us per verification call (split + combine)",
                      "rows": rows}), flush=True)


def phase_trace(layers=8, reps=3):
    """Per-workgroup phase timestamps of the 128K verification call (one-call form's split kernel,
    host-planned, with collection) from the measurement build libvegas_trace.so: start, end of the
    block loop and end of every split workgroup, the CU it ran on (XCD, shader engine, CU ids) and its
    (sequence, split, KV head); `layers` layers, `reps` calls each after a warm-up, with KV head g on
    the workgroups w = g (mod Hkv) (which the dispatcher deals to XCD g) and again with the KV heads
    rotated over the XCDs.  Prints one JSON line of summaries."""
    import ctypes
    import numpy as np
    import torch
    from verification_guided_sparse_verify_amd import build as B
    from verification_guided_sparse_verify_amd import vegas as V
    from verification_guided_sparse_verify_amd import workloads as W
    from verification_guided_sparse_verify_amd.step import LayerStep

    V._lib = None
    V.LIB_PATH = B.TRACE_LIB
    L = V.lib()
    L.vegas_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.vegas_trace_set_rotation.argtypes = [ctypes.c_int]
    wl = W.named_workload(2)
    steps = []
    for layer in range(layers):
        inp = W.make_inputs(wl, seed=0, device="cuda", layer=layer)
        steps.append(LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                               wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts))
    torch.cuda.synchronize()
    out = {"phase_trace": wl.name, "layers": layers, "calls_per_layer": reps,
           "call": "vegas_verify_attn_hostplan with collection (split kernel; libvegas_trace.so)",
           "clock": "wall_clock64, 100 MHz", "mappings": {}}
    buf = np.zeros(4096 * 8, np.uint64)
    for rotate in (0, 1):
        assert L.vegas_trace_set_rotation(rotate) == 0
        recs = []
        for rep in range(reps + 1):
            for st in steps:
                st.verify(collect=True, host_plan=True)
                torch.cuda.synchronize()
                assert L.vegas_trace_read(buf.ctypes.data, buf.nbytes) == 0
                if rep > 0:
                    recs.append(buf.reshape(4096, 8)[:256].astype(np.int64).copy())
        loop, end, start, keys = [], [], [], []
        call_end = []
        for r in recs:
            t0 = r[:, 0].min()
            loop.append((r[:, 1] - r[:, 0]) / 100.0)
            end.append((r[:, 2] - t0) / 100.0)
            start.append((r[:, 0] - t0) / 100.0)
            call_end.append(float(((r[:, 2] - t0) / 100.0).max()))
            keys.append(r)
        loop, end, start = np.concatenate(loop), np.concatenate(end), np.concatenate(start)
        allr = np.concatenate(keys)
        xcc = allr[:, 4] & 15
        cu = ((allr[:, 3] >> 8) & 15) + 16 * ((allr[:, 3] >> 12) & 1) + 32 * ((allr[:, 3] >> 13) & 7) + 256 * xcc
        wgs = np.tile(np.arange(256), len(recs))

        def means(key):
            return {int(k): round(float(loop[key == k].mean()), 1) for k in np.unique(key)}

        def split_half(ids):
            a, b = [], []
            for k in np.unique(ids):
                v = loop[ids == k]
                if len(v) >= 4:
                    a.append(v[0::2].mean())
                    b.append(v[1::2].mean())
            return round(float(np.corrcoef(a, b)[0, 1]), 3)

        pct = lambda x: [round(float(v), 1) for v in np.percentile(x, [0, 10, 50, 90, 100])]
        out["mappings"]["kv_heads_rotated_over_xcds" if rotate else "kv_head_g_on_xcd_g"] = {
            "block_loop_us_p0_p10_p50_p90_max": pct(loop),
            "workgroup_end_us_p0_p10_p50_p90_max": pct(end),
            "last_workgroup_end_us_mean_over_calls": round(float(np.mean(call_end)), 1),
            "last_start_us_max": round(float(start.max()), 2),
            "block_loop_mean_us_by_kv_head": means(allr[:, 7]),
            "block_loop_mean_us_by_xcd": means(xcc),
            "block_loop_mean_us_by_split": means(allr[:, 6]),
            "block_loop_mean_us_by_sequence": means(allr[:, 5]),
            "split_half_correlation_per_workgroup": split_half(wgs),
            "split_half_correlation_per_cu": split_half(cu),
        }
    L.vegas_trace_set_rotation(0)
    print(json.dumps(out), flush=True)


def accept_bench(reps=50):
    """Time vegas_spec_accept on seeded synthetic distributions; one JSON line.  Bytes: the one
    or two vocabulary rows each sequence reads for its draw, plus the tested draft entries."""
    import torch
    from verification_guided_sparse_verify_amd import workloads as W
    from verification_guided_sparse_verify_amd import vegas as V

    rows = []
    for B, gamma, vocab in ((4, 5, 151936), (16, 3, 201088)):
        inp = W.make_accept_inputs(B, gamma, vocab, seed=0, device="cuda:0")
        n = torch.empty(B, dtype=torch.int32, device="cuda:0")
        t = torch.empty(B, dtype=torch.int32, device="cuda:0")
        ws = torch.empty(V.vegas_spec_accept_workspace_size(B, vocab), dtype=torch.uint8, device="cuda:0")
        call = lambda: V.vegas_spec_accept(B, gamma, vocab, inp["p"], inp["q"], inp["draft"], inp["u_accept"],
                                           inp["u_sample"], n, t, ws)
        call()
        torch.cuda.synchronize()
        nacc = n.cpu()
        rows_read = sum(2 if int(k) < gamma else 1 for k in nacc)
        nbytes = rows_read * vocab * 4 + B * gamma * (4 + 4 + 4 + 4)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        rows.append({"batch": B, "gamma": gamma, "vocab": vocab, "us_per_call": round(us, 2),
                     "bytes_per_call": nbytes, "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "accepted": nacc.tolist()})
    print(json.dumps({"accept_bench": rows}), flush=True)


def copy_calibration(nbytes):
    """A plain device-to-device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                      "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, help="0-based workload index (default: 128K Qwen3-8B step)")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (profiling runs only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the measured streaming-read ceiling (4 GiB read by a plain kernel)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time verification and selection as two library calls on one stream")
    ap.add_argument("--single-stream", action="store_true",
                    help="time verification and selection as one library call on the launch stream (by default "
                         "a workload of several layers runs the selection's last steps of layer l on a second "
                         "stream beside the verification of layer l+1; the single-stream figure is reported in "
                         "any case)")
    ap.add_argument("--no-step-sync", action="store_true",
                    help="let the host queue the next step before the GPU has finished the previous one (by "
                         "default a step of several layers, one decoding iteration, ends with a synchronisation: "
                         "the host-planned calls of the next iteration take host copies of sequence lengths that "
                         "depend on this iteration's accepted tokens)")
    ap.add_argument("--kv-offset", type=int, default=None,
                    help="byte offset of each layer's V cache from its K cache modulo 2 MB (default: the "
                         "workload generator's KV_OFFSET_BYTES; 0 puts them at the same offset, as two plain "
                         "allocations usually are)")
    ap.add_argument("--kv-gap", type=int, default=None,
                    help="whole bytes (a multiple of 2 MB) between the end of each layer's K cache, rounded "
                         "up to 2 MB, and its V cache, which share one allocation (default: the workload "
                         "generator's KV_GAP_BYTES)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--page-size", type=int, default=0,
                    help="keep every layer's KV cache as a randomly permuted page pool of this page size and "
                         "run the paged entry points (0: contiguous cache)")
    ap.add_argument("--selection", choices=("vegas", "streaming"), default="vegas",
                    help="vegas: verification-guided selection (the method); streaming: query-agnostic "
                         "sinks + recent tokens with the same budget, no collection (a baseline)")
    ap.add_argument("--collect-sweep", action="store_true",
                    help="only time verification of one layer with collection off, Collect-2-Query and "
                         "all rows, over gamma")
    ap.add_argument("--accept-bench", action="store_true",
                    help="only time the speculative-sampling acceptance step (batch 4, gamma 5, "
                         "Qwen3 vocabulary 151936, and batch 16, gamma 3, gpt-oss vocabulary 201088)")
    ap.add_argument("--device-plan", action="store_true",
                    help="time the entry points that plan splits on the device (default: the *_hostplan entry "
                         "points, which take host copies of the offsets; same results)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="only record per-workgroup phase timestamps of the 128K verification call with the "
                         "measurement build libvegas_trace.so and print their summary")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a device copy of BYTES bytes three times (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    if args.kv_offset is not None:
        if args.kv_offset < 0 or args.kv_offset % 16:
            print("bench.py: --kv-offset must be a non-negative multiple of 16", file=sys.stderr)
            sys.exit(2)
        from verification_guided_sparse_verify_amd import workloads as W
        W.KV_OFFSET_BYTES = args.kv_offset
    if args.kv_gap is not None:
        if args.kv_gap < 0 or args.kv_gap % (2 << 20):
            print("bench.py: --kv-gap must be a non-negative multiple of 2 MB", file=sys.stderr)
            sys.exit(2)
        from verification_guided_sparse_verify_amd import workloads as W
        W.KV_GAP_BYTES = args.kv_gap
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.accept_bench:
        accept_bench()
        return
    if args.phase_trace:
        phase_trace(layers=args.layers or 8)
        return

    import torch
    from verification_guided_sparse_verify_amd import workloads as W
    from verification_guided_sparse_verify_amd import vegas as V
    from verification_guided_sparse_verify_amd.step import LayerStep

    if not os.path.exists(V.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    wl = W.named_workload(args.workload)
    if args.collect_sweep:
        collect_sweep(wl)
        return
    layers = args.layers if args.layers is not None else wl.layers
    dev = "cuda:0"
    cpu_leg = not args.no_cpu_baseline and not args.page_size and args.selection == "vegas"
    t_gen = time.perf_counter()
    layer_inputs, steps = [], []
    for layer in range(layers):
        inp = W.make_inputs(wl, seed=0, device=dev, layer=layer)
        paged = None
        if args.page_size:
            paged = W.page_cache(wl, inp, args.page_size, seed=layer, drop_contiguous=True)
        layer_inputs.append(inp)
        steps.append(LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma,
                               wl.seqlens, wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts, paged=paged,
                               selection=args.selection))
        if layer % 6 == 5:
            torch.cuda.synchronize()
            print(f"# generated layer {layer + 1}/{layers}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    print(f"# generated {layers} layers in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    # Host-planned entry points (host copies of the offsets) unless asked otherwise; they
    # cover the contiguous cache.
    host_plan = not args.device_plan and not args.page_size
    bound = [st.bind(stream, host_plan=host_plan) for st in steps]     # ctypes arguments converted once
    # Verification and selection as one library call where the path allows it.
    fused = steps[0].fusable and not args.separate_calls
    fused_calls = [st.bind_fused(stream, host_plan=host_plan) for st in steps] if fused else None
    # The one call in two halves, the selection of layer l (keys, candidates, write) on a second
    # stream beside the verification of layer l+1: the selected positions are used only by the
    # drafting passes, which wait for each layer's selection, while layer l+1's verification
    # needs only layer l's output, complete when the first half ends.
    overlap = fused and host_plan and layers > 1 and not args.single_stream
    # The second halves go to the side stream in groups of SEL_GROUP layers, each group after its
    # last layer's first half: every cross-stream event costs the launch stream ~1 us, and the
    # selections are needed only by the drafting passes (interleaved in one process, 128K step, µs
    # per layer-step: 464.7 with a group per layer, 459.9 with groups of 4, 458.7 of 6, 458.2 of 9,
    # 458.7 of 12; 449.6 with no selection work at all).
    SEL_GROUP = 9
    side = torch.cuda.Stream() if overlap else None              # default priority, as the launch stream
    begin_calls = [st.bind_fused(stream, part="begin") for st in steps] if overlap else None
    end_calls = [st.bind_fused(side, part="end") for st in steps] if overlap else None
    verified = [torch.cuda.Event() for _ in steps] if overlap else None
    selected = [torch.cuda.Event() for _ in steps] if overlap else None

    def one_step(head_events=None, call_events=None, single_stream=False):
        """One speculative iteration: verify + select on every layer, then gamma drafting
        passes over every layer.  head_events: list receiving an event pair around every
        verify (separate calls) or verify+select (one call, or its first half with the
        second half on the second stream); call_events: dict receiving event pairs around every
        call of the separate-call path; single_stream: the one call on the launch stream."""
        def timed(kind, fn, sink):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            sink[kind].append((a, b))

        halves = overlap and not single_stream and call_events is None
        for li, (verify, verify_plain, select, _) in enumerate(bound):
            if call_events is not None:
                # separate calls, then plain verification and the one call on the same layer, so that
                # the collection + selection overhead compares calls made in the same conditions
                timed("verify", verify, call_events)
                timed("select", select, call_events)
                timed("plain", verify_plain, call_events)
                if fused:
                    timed("one_call", fused_calls[li], call_events)
                continue
            head = begin_calls[li] if halves else (fused_calls[li] if fused else verify)
            if head_events is not None:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                head()
                b.record(stream)
                head_events.append((a, b))
            else:
                head()
            if halves:
                # the second halves of a group of layers, once the group's last first half is done
                if (li + 1) % SEL_GROUP == 0 or li == layers - 1:
                    verified[li].record(stream)
                    side.wait_event(verified[li])
                    for lj in range(li - li % SEL_GROUP, li + 1):
                        end_calls[lj]()
                    selected[li].record(side)
            elif not fused:
                select()
        for j in range(wl.n_drafts):
            for li, (_, _, _, drafts) in enumerate(bound):
                if halves and j == 0 and li % SEL_GROUP == 0:
                    # the first drafting pass needs the selections of the group of layer li
                    stream.wait_event(selected[min(li + SEL_GROUP - 1, layers - 1)])
                if call_events is not None:
                    timed("draft", drafts[j], call_events)
                else:
                    drafts[j]()

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    # The timed region runs the steps alone: timing events around every call would add ~7 us
    # per layer-step (each timed event waits for the work before it); the per-call durations
    # come from instrumented steps after it.
    # A step of several layers is one decoding iteration: the host plans the next iteration's calls
    # from sequence lengths that depend on this iteration's accepted tokens, so it waits for the
    # step to finish before queueing the next one. (A one-layer workload stands for one layer of
    # such an iteration, whose next layer would follow without a host round trip.)
    step_sync = layers > 1 and not args.no_step_sync

    def timed_steps(n, **kw):
        t = time.perf_counter()
        for _ in range(n):
            one_step(**kw)
            if step_sync:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        return time.perf_counter() - t

    elapsed = timed_steps(args.steps)
    # The same steps with the host queueing ahead of the GPU, for comparison.
    elapsed_ahead = None
    if step_sync:
        t1 = time.perf_counter()
        for _ in range(args.steps):
            one_step()
        torch.cuda.synchronize()
        elapsed_ahead = time.perf_counter() - t1

    # Instrumented steps of the same schedule: events around every verification (or
    # verification + selection) call.
    head_pairs = []
    for _ in range(max(2, 12 // layers)):
        one_step(head_events=head_pairs)
    torch.cuda.synchronize()

    # The one call on the launch stream alone, for comparison with the two-stream schedule.
    single_ms, single_heads = None, []
    if overlap:
        one_step(single_stream=True)
        torch.cuda.synchronize()
        n_single = max(3, args.steps // 2)
        single_ms = timed_steps(n_single, single_stream=True) * 1e3 / n_single
        one_step(head_events=single_heads, single_stream=True)   # the one call's own duration
        torch.cuda.synchronize()

    # Per-call breakdown, outside the timed region: more steps with events around every call.
    call_pairs = {"verify": [], "select": [], "draft": [], "plain": [], "one_call": []}
    for _ in range(max(2, 12 // layers)):          # at least a dozen calls of each kind
        one_step(call_events=call_pairs)
    torch.cuda.synchronize()
    per = {k: [a.elapsed_time(b) * 1e3 for a, b in v] for k, v in call_pairs.items() if v}   # microseconds
    plain_us = statistics.fmean(per.pop("plain"))
    one_call_us = statistics.fmean(per.pop("one_call")) if fused else None
    mean = {k: statistics.fmean(v) for k, v in per.items()}
    med = {k: statistics.median(v) for k, v in per.items()}

    def p10_p90(xs):
        q = statistics.quantiles(xs, n=10, method="inclusive") if len(xs) > 1 else [xs[0]] * 9
        return q[0], q[-1]
    pct = {k: p10_p90(v) for k, v in per.items()}
    head_us = [a.elapsed_time(b) * 1e3 for a, b in head_pairs]
    if fused:
        # The timed region runs verification + selection as one call (or its first half); the
        # verification kernels' own duration comes from the separate-call steps of the breakdown.
        verify_us = per["verify"]
        head_key = "verify_select_first_half" if overlap else "verify_select"
        mean[head_key] = statistics.fmean(head_us)
        med[head_key] = statistics.median(head_us)
        pct[head_key] = p10_p90(head_us)
        if overlap:
            one = [a.elapsed_time(b) * 1e3 for a, b in single_heads]
            mean["verify_select"] = statistics.fmean(one)
            med["verify_select"] = statistics.median(one)
            pct["verify_select"] = p10_p90(one)
    else:
        verify_us = head_us
    verify_mean = statistics.fmean(verify_us)

    ms_per_step = elapsed * 1e3 / args.steps
    us_layer_step = ms_per_step * 1e3 / layers
    ab = algorithmic_bytes(wl)
    step_gbps = ab["layer_step"] / (us_layer_step * 1e-6) / 1e9
    verify_gbps = ab["verify"] / (verify_mean * 1e-6) / 1e9
    traffic = read_traffic("attn_split_verify_qwen3_8b_128k_pmc.txt", "hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(us_layer_step, 2),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) K/V with planted heavy hitters, sinks and recency band)",
        "config": {
            "workload": wl.name if layers == wl.layers else f"{wl.name} (layers={layers})",
            "batch": wl.batch, "layers": layers, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "prefix_lens": sorted(set(wl.prefix_lens)) if len(set(wl.prefix_lens)) <= 2 else "ragged",
            "gamma": wl.gamma, "k_per_seq": wl.k_per_seq if len(set(wl.k_per_seq)) > 1 else wl.k_per_seq[0],
            "kv_cache_bytes": wl.total_kv * wl.num_kv_heads * wl.head_dim * (2 if wl.dtype == "bf16" else 4) * 2 * layers,
            "order": "verify+select over all layers, then gamma drafting passes over all layers",
            "kv_cache": (f"paged, {args.page_size}-token pages in a randomly permuted pool" if args.page_size
                         else f"contiguous varlen, each layer's K and V in one allocation, V {W.KV_GAP_BYTES + W.KV_OFFSET_BYTES} B "
                           f"past K's end rounded up to 2 MB"),
            "selection": ("verification-guided (Collect-2-Query + exact top-k)" if args.selection == "vegas"
                          else "query-agnostic: 4 sinks + most recent tokens, same k, no collection"),
        },
        "layer_step_gbps": round(step_gbps, 1),
        "layer_step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "per_call_us": {k: {"mean": round(mean[k], 2), "median": round(med[k], 2),
                            "p10": round(pct[k][0], 2), "p90": round(pct[k][1], 2)} for k in mean},
        "collect_select_overhead_vs_plain_verify": None,
        "roofline": {
            "kernel": "verify: attn_split_kernel (+ attn_combine) per layer",
            "bound": "hbm",
            "achieved": round(verify_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(verify_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["verify"],
            "avg_launch_us": round(verify_mean, 2),
            "launches_timed": len(verify_us),
            "timed_in": ("separate-call breakdown steps after the timed region (which runs verification "
                         "and selection as one call, or its two halves)" if fused else
                         "instrumented steps of the timed schedule after the timed region (which runs without "
                         "timing events)"),
        },
    }
    sfx = "_hostplan" if host_plan else ""
    if overlap:
        result["config"]["calls"] = ("vegas_verify_select_begin_hostplan per layer on the launch stream, "
                                     "vegas_verify_select_end_hostplan of layers 4m..4m+3 on a second stream after "
                                     "layer 4m+3's first half, beside the next layers; then gamma x "
                                     "vegas_sparse_decode_attn_hostplan per layer")
        result["layer_step_single_stream_us"] = round(single_ms * 1e3 / layers, 2)
        result["layer_step_single_stream_calls"] = ("vegas_verify_select_hostplan + gamma x "
                                                    "vegas_sparse_decode_attn_hostplan per layer, one stream")
    else:
        result["config"]["calls"] = (f"vegas_verify_select{sfx} + gamma x vegas_sparse_decode_attn{sfx} per layer"
                                     if fused else
                                     f"verify{sfx}, select and gamma sparse-decode{sfx} calls per layer")
    result["config"]["split_plan"] = ("host (host copies of the offsets, computed per call)" if host_plan
                                      else "device")
    result["config"]["host_sync"] = ("after every step (one decoding iteration): the next iteration's host plans "
                                      "need its accepted lengths" if step_sync else "none between steps")
    if elapsed_ahead is not None:
        result["layer_step_host_ahead_us"] = round(elapsed_ahead * 1e6 / args.steps / layers, 2)

    # Plain verification (collection off) was timed in the breakdown steps, layer by layer next to
    # the separate calls and the one call, for the collection + select overhead.
    result["plain_verify_us"] = round(plain_us, 2)
    separate = (mean["verify"] + mean["select"]) / plain_us - 1
    result["collect_select_overhead_vs_plain_verify"] = round(
        (one_call_us if fused else verify_mean + mean["select"]) / plain_us - 1, 4)
    if fused:
        result["one_call_breakdown_us"] = round(one_call_us, 2)
    result["collect_select_overhead_separate_calls"] = round(separate, 4)
    # Achieved algorithmic bandwidth of each of the three calls (per-call means of the breakdown).
    result["per_call_gbps"] = {
        kind: {"algorithmic_bytes": ab[kind], "gbps": round(ab[kind] / (mean[kind] * 1e-6) / 1e9, 1),
               "frac_of_peak": round(ab[kind] / (mean[kind] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        for kind in ("verify", "select", "draft")}

    if not args.no_stream_ceiling:
        ceiling = stream_read_ceiling()
        result["stream_read_ceiling"] = ceiling
        if ceiling:
            result["roofline"]["frac_of_stream_ceiling"] = round(verify_gbps / ceiling["gbps"], 4)
            result["layer_step_frac_of_stream_ceiling"] = round(step_gbps / ceiling["gbps"], 4)
        if not args.page_size:
            gceil = gather_read_ceiling(wl, layer_inputs, steps)
            result["gather_read_ceiling"] = gceil
            if gceil:
                result["per_call_gbps"]["draft"]["frac_of_gather_ceiling"] = round(
                    result["per_call_gbps"]["draft"]["gbps"] / gceil["gbps"], 4)

    floor = launch_floor()
    if floor:
        result["dependent_launch_floor"] = floor
        if fused:
            # the one call runs the combine with the selection's first step, then two selection
            # launches (candidates, write): two kernel boundaries more than plain verification
            f2 = 2 * floor["256_workgroups_64kb_lds"]
            result["collect_select_launch_floor_us"] = round(f2, 2)
            result["collect_select_launch_floor_vs_plain_verify"] = round(f2 / plain_us, 4)

    if cpu_leg:
        result["cpu_baseline"] = cpu_baseline(wl, layer_inputs, args.cpu_seconds)
        result["cpu_baseline"]["tiny_single_thread"] = tiny_single_thread_oracle()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
