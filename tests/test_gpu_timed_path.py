"""Oracle parity of exactly the calls bench.py times, at the workloads' full sizes: the
one-call verification + selection and the drafting calls with host copies of the offsets
(vegas_verify_select_hostplan, vegas_sparse_decode_attn_hostplan), the split plan the benchmark
runs (the balanced plan for the ragged batch), checked against the CPU oracle on every sequence
of the batch.  Each case's worst errors go to gpurun_out/parity_margins.json beside its
tolerances."""
import pytest
import torch

from verification_guided_sparse_verify_amd import workloads as W
from verification_guided_sparse_verify_amd import vegas as V
from verification_guided_sparse_verify_amd.step import LayerStep

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from parity_util import check_layer, log, record_margins


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _timed_layer(wl: W.Workload, layer: int):
    """One layer through the calls bench.py times for this workload: with several layers the one
    call in two halves, the second on another stream; with one layer the one call."""
    inp = W.make_inputs(wl, seed=0, device="cuda", layer=layer)
    st = LayerStep(inp, wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.gamma, wl.seqlens,
                   wl.k_per_seq, wl.scale, n_drafts=wl.n_drafts)
    st.run(fused=True, host_plan=True, select_stream=torch.cuda.Stream() if wl.layers > 1 else None)
    torch.cuda.synchronize()
    return inp, st


# workload index, layer (the 36-layer workload draws every layer with its own seed)
TIMED = [(1, 0), (2, 0), (2, 35), (3, 0), (4, 0)]


@pytest.mark.parametrize("case", TIMED, ids=lambda c: f"workload{c[0]}-layer{c[1]}")
def test_benchmarked_calls_match_oracle_on_every_sequence(case):
    i, layer = case
    wl = W.named_workload(i)
    log(f"case: timed path, {wl.name}, layer {layer}")
    inp, st = _timed_layer(wl, layer)
    balanced, wgs = V.vegas_verify_hostplan_info(st.shape, wl.gamma, st.max_seqlen, st.total_kv, st.host)
    log(f"  split plan: {'balanced' if balanced else 'per sequence'}, {wgs} workgroups per KV head")
    if i == 4:
        assert balanced          # the ragged batch takes the balanced plan: checked directly here
    worst = check_layer(wl, inp, st)
    record_margins(f"timed-workload{i}-layer{layer}", wl, worst, range(wl.batch))
