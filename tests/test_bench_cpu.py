"""bench.py's contract on the CPU: the algorithmic bytes it divides by (written out here from the
shapes), its refusal of more than one GPU and of malformed cache placement flags, and the filter
that keys the counter summaries to the product kernels' code."""
import os
import subprocess
import sys

import bench
from verification_guided_sparse_verify_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_qwen3_8b_shapes():
    """Per call type, the bytes the method must move: K and V read once for all query rows, Q read
    and O written, the collected scores written (verify) and read (select), the selected list
    written, and per drafting call the selected rows' K and V of every KV head plus the list, q and o."""
    # 128K step: 4 sequences of 131072 + 6 rows, 8 KV heads, D 128, bf16; 32/8 heads, gamma 5, k 6553
    rows, hkv, d, es = 4 * (131072 + 6), 8, 128, 2
    kv = rows * hkv * d * es * 2
    qo = 4 * 6 * 32 * d * es * 2
    scores = hkv * 4 * 131072 * 4
    ab = bench.algorithmic_bytes(W.named_workload(2))
    assert ab["verify"] == kv + qo + scores == 2_164_752_384
    assert ab["select"] == scores + 4 * 6553 * 4
    assert ab["draft"] == 4 * 6553 * hkv * d * es * 2 + 4 * 6553 * 4 + 4 * 32 * d * es * 2
    assert ab["layer_step"] == ab["verify"] + ab["select"] + 5 * ab["draft"]
    # 32K layer: gamma 4, k 1638 per sequence, four drafting calls
    ab1 = bench.algorithmic_bytes(W.named_workload(1))
    assert ab1["verify"] == 4 * (32768 + 5) * hkv * d * es * 2 + 4 * 5 * 32 * d * es * 2 + hkv * 4 * 32768 * 4
    assert ab1["draft"] == 4 * 1638 * hkv * d * es * 2 + 4 * 1638 * 4 + 4 * 32 * d * es * 2
    assert ab1["layer_step"] == ab1["verify"] + ab1["select"] + 4 * ab1["draft"]
    assert round(ab1["layer_step"] / 1e6, 1) == 653.4


def test_bench_refuses_more_than_one_gpu():
    """One GPU only: --gpus above 1 exits with status 2 and says so, before touching a device."""
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    assert run.returncode == 2
    assert "one GPU only" in run.stderr and "--gpus 2" in run.stderr
    assert run.stdout == ""


def test_bench_rejects_bad_kv_placement_arguments():
    """--kv-offset takes a non-negative multiple of 16 bytes and --kv-gap a non-negative multiple of
    2 MB; anything else exits with status 2 and says which, before touching a device."""
    for flag, value, msg in (("--kv-offset", "8", "--kv-offset must be"), ("--kv-offset", "-16", "--kv-offset must be"),
                             ("--kv-gap", "1000", "--kv-gap must be"), ("--kv-gap", str(3 << 20), "--kv-gap must be")):
        run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), flag, value], capture_output=True,
                             text=True, timeout=300, cwd=ROOT)
        assert run.returncode == 2, (flag, value, run.stderr)
        assert msg in run.stderr and run.stdout == ""


def test_counter_key_ignores_comments_and_the_trace_build():
    """The counter summaries are keyed by a hash of the product code: comments, blank lines and the
    measurement-only trace branches do not enter it, the trace branches' #else branches do."""
    text = """int a = 1;  // comment
/* block
   comment */
#ifdef VEGAS_PHASE_TRACE
int traced = 2;
#else
int plain = 3;
#endif

#ifdef OTHER
int other = 4;
#endif
"""
    assert bench.product_code_lines(text) == ["int a = 1;", "int plain = 3;", "#ifdef OTHER", "int other = 4;",
                                              "#endif"]
    assert len(bench.kernel_source_hash()) == 16
