"""vegas_sparse_decode_attn_noalloc (drafting on the library's static scratch) against
vegas_sparse_decode_attn with a caller workspace, through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to the workspace call on the same input (same
kernels) and within the output tolerance of the oracle; with and without host offsets."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from verification_guided_sparse_verify_amd import workloads as W
from verification_guided_sparse_verify_amd import vegas as V

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from parity_util import ATOL, _seq_host, log, run_layer


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


CASES = [
    # dtype, batch, Hq, Hkv, D, gamma, prefix lengths, selection ratio (the second call is the smaller one)
    ("bf16", 4, 32, 8, 128, 5, [20000, 9000, 30000, 500], Fraction(20, 100)),
    ("bf16", 2, 16, 4, 64, 2, [3000, 700], Fraction(5, 100)),
]


def _draft_both_ways(case, host_plan: bool):
    dtype, B, hq, hkv, d, gamma, prefixes, ratio = case
    wl = W.custom_workload(dtype, B, hq, hkv, d, gamma, prefixes, ratio=ratio)
    inp, st = run_layer(wl, seed=31)
    host = st.host if host_plan else None
    q = inp["draft_q"][0]
    ref = torch.full_like(q, 7.0)
    if host_plan:
        V.vegas_sparse_decode_attn_hostplan(st.shape, q, inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv,
                                            st.indices, inp["cu_k"], st.max_k, ref, st.workspace, st.host)
    else:
        V.vegas_sparse_decode_attn(st.shape, q, inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv, st.indices,
                                   inp["cu_k"], st.max_k, ref, st.workspace)
    got = torch.full_like(q, 5.0)
    V.vegas_sparse_decode_attn_noalloc(st.shape, q, inp["k"], inp["v"], inp["cu_seqlens_k"], wl.total_kv, st.indices,
                                       inp["cu_k"], st.max_k, got, host=host)
    torch.cuda.synchronize()
    return wl, inp, st, ref, got


@pytest.mark.parametrize("host_plan", [False, True], ids=["device-plan", "host-plan"])
def test_noalloc_drafting_equals_workspace_call(host_plan):
    assert V.vegas_noalloc_scratch_bytes() == 16 << 20
    for case in CASES:       # two calls in a row, the second smaller
        wl, inp, st, ref, got = _draft_both_ways(case, host_plan)
        need = V.vegas_sparse_decode_workspace_size(st.shape, st.max_k)
        log(f"case: noalloc {wl.name} L={wl.prefix_lens} host_plan={host_plan} scratch need {need} B")
        assert need <= V.vegas_noalloc_scratch_bytes()
        assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
        cuk = wl.cu_k()
        for b in range(wl.batch):
            _, k, v, cu1 = _seq_host(inp, wl, b)
            t = st.indices[cuk[b]:cuk[b + 1]].cpu().numpy()
            d_ref = oracle.sparse_decode_attn(W.host_bits(inp["draft_q"][0][b:b + 1]), k, v, cu1, t,
                                              np.array([0, len(t)], np.int32), wl.scale)
            err = float(np.abs(got[b:b + 1].float().cpu().numpy() - d_ref).max())
            assert err <= ATOL[wl.dtype], (b, err)


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A call whose workspace would exceed the static scratch returns VEGAS_ERR_UNSUPPORTED with the
    sizes in the message, and launches nothing."""
    shape = V.attn_shape(V.VEGAS_DTYPE_F32, 1024, 256, 16, 128, 0.125)
    need = V.vegas_sparse_decode_workspace_size(shape, 100000)
    assert need > V.vegas_noalloc_scratch_bytes()
    fake = 0x100000
    rc = V.lib().vegas_sparse_decode_attn_noalloc(V.ctypes.byref(shape), fake, fake, fake, fake, 10 ** 6, fake, fake,
                                                  100000, fake, None, None)
    assert rc == V.VEGAS_ERR_UNSUPPORTED
    assert V.lib().vegas_last_error_message().decode().startswith(f"this call needs {need} bytes of scratch")
