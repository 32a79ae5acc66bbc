"""Host-side contract of libvegas.so, no GPU needed: the library loads, exports
every entry point the header declares, sizes workspaces, and rejects bad
arguments before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def V():
    from verification_guided_sparse_verify_amd import vegas
    if not os.path.exists(vegas.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    vegas.lib()
    return vegas


def header_functions():
    text = open(os.path.join(ROOT, "include", "vegas.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vegas_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(V):
    names = header_functions()
    assert len(names) >= 9
    nm = subprocess.run(["nm", "-D", "--defined-only", V.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(ln.split()[-1] for ln in nm.splitlines() if ln.strip())
    for n in names:
        assert n in exported, n
        assert hasattr(V.lib(), n)
    assert set(V.EXPORTED) == set(names)


def test_abi_version_and_status_strings(V):
    assert V.vegas_abi_version() == 1
    assert V.status_string(0) == "VEGAS_OK"
    assert V.status_string(3) == "VEGAS_ERR_WORKSPACE_TOO_SMALL"


def shape(V, **kw):
    p = dict(dtype=V.VEGAS_DTYPE_BF16, batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
             softmax_scale=128 ** -0.5)
    p.update(kw)
    return V.attn_shape(p["dtype"], p["batch"], p["num_q_heads"], p["num_kv_heads"], p["head_dim"],
                        p["softmax_scale"])


def test_workspace_sizes(V):
    s = shape(V)
    a = V.vegas_verify_workspace_size(s, 4, 32773)
    b = V.vegas_verify_workspace_size(s, 4, 131078)
    assert 0 < a <= b
    assert V.vegas_select_workspace_size(4, 8, 4, 32773, 4 * 32773) >= 4 * 32773 * 12
    assert V.vegas_sparse_decode_workspace_size(s, 1638) > 0
    assert V.vegas_sparse_decode_workspace_size(s, 0) >= 0


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), 2),
    (dict(dtype=7), 2),
    (dict(num_q_heads=30), 1),
    (dict(batch=0), 1),
    (dict(softmax_scale=0.0), 1),
    (dict(softmax_scale=float("nan")), 1),
])
def test_bad_shapes_rejected(V, kw, code):
    with pytest.raises(V.VegasError) as e:
        V.vegas_verify_workspace_size(shape(V, **kw), 4, 1000)
    assert e.value.status == code


def test_gamma_limits(V):
    with pytest.raises(V.VegasError) as e:
        V.vegas_verify_workspace_size(shape(V), 32, 1000)
    assert e.value.status == 1
    with pytest.raises(V.VegasError) as e:       # (gamma+1)*G = 17*4 > 64 rows per KV head
        V.vegas_verify_workspace_size(shape(V), 16, 1000)
    assert e.value.status == 2


FAKE = 0x100000  # a 16-byte aligned non-NULL value; validation fails before any use


def test_verify_argument_errors(V):
    s = shape(V)
    ws = V.vegas_verify_workspace_size(s, 4, 1000)
    L = V.lib()

    def call(**kw):
        p = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, maxs=1000, total=4000, mask=1 | 16, scores=FAKE, out=FAKE,
                 ws=FAKE, wsb=ws)
        p.update(kw)
        return L.vegas_verify_attn(ctypes.byref(s), 4, p["q"], p["k"], p["v"], p["cu"], p["maxs"], p["total"],
                                   p["mask"], p["scores"], p["out"], p["ws"], p["wsb"], None)

    def msg():
        return L.vegas_last_error_message().decode()

    assert call(q=None) == 1
    assert "must be non-NULL" in msg()
    assert call(out=FAKE + 4) == 1                       # misaligned
    assert "16-byte aligned" in msg()
    assert call(mask=1 << 5) == 1                        # row 5 does not exist for gamma 4
    assert "rows >= gamma+1 = 5" in msg()
    assert call(scores=None) == 1                        # collection on, no buffer
    assert "scores is NULL" in msg()
    assert call(wsb=ws - 1) == 3
    assert msg() == f"workspace needs {ws} bytes, got {ws - 1}"
    assert call(maxs=3) == 1
    assert "max_seqlen_k 3 < gamma+1" in msg()
    assert call(total=4) == 1
    assert "total_kv 4 < batch*(gamma+1)" in msg()


def test_select_and_decode_argument_errors(V):
    L = V.lib()
    ws = V.vegas_select_workspace_size(2, 8, 3, 100, 200)
    assert L.vegas_select_topk(2, 8, 3, None, FAKE, 100, 200, FAKE, FAKE, FAKE, ws, None) == 1
    assert L.vegas_select_topk(2, 8, 3, FAKE, FAKE, 100, 200, FAKE, FAKE, FAKE, ws - 1, None) == 3
    assert L.vegas_select_topk(2, 8, 40, FAKE, FAKE, 100, 200, FAKE, FAKE, FAKE, ws, None) == 1
    s = shape(V)
    dws = V.vegas_sparse_decode_workspace_size(s, 50)
    assert L.vegas_sparse_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 200, FAKE, None, 50, FAKE, FAKE,
                                      dws, None) == 1
    assert L.vegas_sparse_decode_attn(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 200, FAKE, FAKE, 50, FAKE, FAKE,
                                      dws - 1, None) == 3
    msg = L.vegas_last_error_message().decode()
    assert "workspace" in msg


def test_product_code_never_imports_oracle():
    """The GPU path and its binding share nothing with the oracle."""
    pkg = os.path.join(ROOT, "verification_guided_sparse_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "vegas_oracle" not in text, f


def test_paged_argument_errors(V):
    s = shape(V)
    L = V.lib()
    ws = V.vegas_verify_paged_workspace_size(s, 4, 1000, 16)
    assert ws >= V.vegas_verify_workspace_size(s, 4, 1000)
    assert V.vegas_verify_paged_workspace_size(s, 4, 1000, 1) >= ws     # tiny pages cap the split length
    for bad in (3, 512, -1):
        with pytest.raises(V.VegasError) as e:
            V.vegas_verify_paged_workspace_size(s, 4, 1000, bad)
        assert e.value.status == 2

    def verify(pages, wsb=ws):
        return L.vegas_verify_attn_paged(ctypes.byref(s), 4, FAKE, FAKE, FAKE, pages, FAKE, 1000, 4000, 1 | 16,
                                         FAKE, FAKE, FAKE, wsb, None)

    assert verify(None) == 1
    assert verify(ctypes.byref(V.PagedKV(FAKE, 62, 16, 100))) == 1     # 62 pages of 16 < 1000 positions
    assert verify(ctypes.byref(V.PagedKV(None, 63, 16, 100))) == 1     # no block table
    assert verify(ctypes.byref(V.PagedKV(FAKE, 63, 24, 100))) == 2     # not a power of two
    assert verify(ctypes.byref(V.PagedKV(FAKE, 64, 16, 0))) == 1       # empty pool
    assert verify(ctypes.byref(V.PagedKV(FAKE, 64, 16, 100)), ws - 1) == 3
    dws = V.vegas_sparse_decode_workspace_size(s, 50)
    assert L.vegas_sparse_decode_attn_paged(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, 200, FAKE, FAKE, 50,
                                            FAKE, FAKE, dws, None) == 1
    assert L.vegas_sparse_decode_attn_paged(ctypes.byref(s), FAKE, FAKE, FAKE,
                                            ctypes.byref(V.PagedKV(FAKE, 4, 128, 10)), FAKE, 200, FAKE, FAKE, 50,
                                            FAKE, FAKE, dws - 1, None) == 3


def test_local_and_streaming_argument_errors(V):
    s = shape(V)
    L = V.lib()
    ws = V.vegas_verify_local_workspace_size(s, 4, 100000, 128)
    assert ws <= V.vegas_verify_workspace_size(s, 4, 100000)      # the band bounds the splits
    with pytest.raises(V.VegasError):
        V.vegas_verify_local_workspace_size(s, 4, 100000, 0)
    assert L.vegas_verify_attn_local(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, 1000, 4000, 0, FAKE, FAKE, ws,
                                     None) == 1
    assert L.vegas_verify_attn_local(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, 1000, 4000, 128, FAKE, FAKE, 0,
                                     None) == 3
    assert L.vegas_streaming_indices(0, 4, 4, FAKE, 100, FAKE, 10, FAKE, None) == 1
    assert L.vegas_streaming_indices(2, 4, -1, FAKE, 100, FAKE, 10, FAKE, None) == 1
    assert L.vegas_streaming_indices(2, 4, 4, FAKE, 100, FAKE, 10, None, None) == 1


def test_spec_accept_argument_errors(V):
    L = V.lib()
    ws = V.vegas_spec_accept_workspace_size(4, 151936)
    assert ws >= 4 * 38 * 16
    for args, code in [((0, 3, 100), 1), ((2, 32, 100), 1), ((2, 3, 0), 1)]:
        assert L.vegas_spec_accept(*args, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == code
    assert L.vegas_spec_accept(2, 3, 100, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 1
    assert L.vegas_spec_accept(2, 3, 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None) == 1
    assert L.vegas_spec_accept(2, 3, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == 3


def test_verify_select_sizes_and_argument_errors(V):
    s = shape(V)
    L = V.lib()
    need = V.vegas_verify_select_workspace_size(s, 4, 1000, 4000)
    vb = V.vegas_verify_workspace_size(s, 4, 1000)
    sb = V.vegas_select_workspace_size(4, 8, 4, 1000, 4000)
    assert need == (vb + 255) // 256 * 256 + sb

    def call(**kw):
        p = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, maxs=1000, total=4000, mask=1 | 16, cu_k=FAKE, scores=FAKE,
                 idx=FAKE, out=FAKE, ws=FAKE, wsb=need)
        p.update(kw)
        return L.vegas_verify_select(ctypes.byref(s), 4, p["q"], p["k"], p["v"], p["cu"], p["maxs"], p["total"],
                                     p["mask"], p["cu_k"], p["scores"], p["idx"], p["out"], p["ws"], p["wsb"],
                                     None)

    assert call(mask=0) == 1                 # nothing collected, nothing to select from
    assert call(cu_k=None) == 1
    assert call(idx=None) == 1
    assert call(scores=None) == 1
    assert call(q=None) == 1
    assert call(mask=1 << 5) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 1
    assert call(maxs=3) == 1
    with pytest.raises(V.VegasError) as e:   # the selection's own limit on the prefix length
        V.vegas_verify_select_workspace_size(s, 4, 2048 * 4096 + 1, 4 * (2048 * 4096 + 1))
    assert e.value.status == 2


def test_hostplan_offsets_are_checked_before_launch(V):
    """The *_hostplan calls check the host copies of the offsets and launch nothing when they
    are malformed (batch 4, gamma 4: every sequence needs 5 .. max_seqlen_k rows)."""
    s = shape(V)
    L = V.lib()
    need = V.vegas_verify_select_workspace_size(s, 4, 1000, 4000)
    vws = V.vegas_verify_workspace_size(s, 4, 1000)
    dws = V.vegas_sparse_decode_workspace_size(s, 50)
    good_cu, good_k = [0, 1000, 2000, 3000, 4000], [0, 50, 100, 150, 200]

    def vs(cu, cuk, host=True):
        h = V.host_offsets(cu, cuk)
        return L.vegas_verify_select_hostplan(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, 1000, 4000, 1 | 16, FAKE,
                                              FAKE, FAKE, FAKE, FAKE, need, None, ctypes.byref(h) if host else None)

    def va(cu):
        h = V.host_offsets(cu, [0])
        return L.vegas_verify_attn_hostplan(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, 1000, 4000, 0, None, FAKE,
                                            FAKE, vws, None, ctypes.byref(h))

    def dr(cu, cui):
        h = V.host_offsets(cu, cui)
        return L.vegas_sparse_decode_attn_hostplan(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 4000, FAKE, FAKE, 50,
                                                   FAKE, FAKE, dws, None, ctypes.byref(h))

    assert vs(good_cu, good_k, host=False) == 1
    assert vs([0, 1000, 900, 3000, 4000], good_k) == 1          # decreasing
    assert vs([0, 1000, 2000, 3000, 4001], good_k) == 1         # past total_kv
    assert vs([0, 4, 2000, 3000, 4000], good_k) == 1            # fewer rows than gamma + 1
    assert vs([0, 1001, 2000, 3000, 4000], good_k) == 1         # longer than max_seqlen_k
    assert vs(good_cu, [0, 50, 40, 150, 200]) == 1              # cu_k decreasing
    assert va([-1, 1000, 2000, 3000, 4000]) == 1
    assert dr(good_cu, [0, 50, 100, 151, 200]) == 1             # a list longer than max_idx
    assert L.vegas_last_error_message().decode() == "list 2 holds 51 indices, more than max_idx 50"
    assert dr([0, 1000, 2000, 3000, 3000 - 1], [0, 1, 2, 3, 4]) == 1
    assert L.vegas_last_error_message().decode() == "host cu_seqlens_k decreases at 3 (3000 -> 2999)"
    # well-formed host offsets get as far as the workspace check
    assert L.vegas_sparse_decode_attn_hostplan(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 4000, FAKE, FAKE, 50,
                                               FAKE, FAKE, dws - 1, None,
                                               ctypes.byref(V.host_offsets(good_cu, good_k))) == 3


def test_probe_library_exports_and_rejects_bad_arguments(V):
    """libvegas_probe.so (measurement helper of the benchmark) exports what its header declares and
    validates its arguments before launching anything."""
    from verification_guided_sparse_verify_amd import build as B
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "vegas_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(vegas_[a-z_0-9]+)\s*\(", text)))
    assert names == ["vegas_probe_delay", "vegas_probe_gather_read", "vegas_probe_launch_chain",
                     "vegas_probe_stream_read"]
    nm = subprocess.run(["nm", "-D", "--defined-only", B.PROBE_LIB], capture_output=True, text=True).stdout
    assert all(n in nm for n in names)
    fn = ctypes.CDLL(B.PROBE_LIB).vegas_probe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    unit = 32768 * 256
    assert fn(None, unit, 256, FAKE, None) == -1            # no source
    assert fn(FAKE + 4, unit, 256, FAKE, None) == -1        # misaligned
    assert fn(FAKE, unit + 16, 256, FAKE, None) == -1       # not a whole number of slices
    assert fn(FAKE, unit, 0, FAKE, None) == -1              # no workgroups
    assert fn(FAKE, unit, 256, None, None) == -1            # no sink


def test_noalloc_drafting_rejects_calls_beyond_its_scratch(V):
    """The allocation-free drafting entry point checks the call's scratch need against its static
    scratch before touching the device: too large a call returns VEGAS_ERR_UNSUPPORTED with both
    sizes in the message."""
    L = V.lib()
    assert V.vegas_noalloc_scratch_bytes() == 16 << 20
    s = shape(V, dtype=V.VEGAS_DTYPE_F32, batch=1024, num_q_heads=256, num_kv_heads=16)
    need = V.vegas_sparse_decode_workspace_size(s, 100000)
    assert need > V.vegas_noalloc_scratch_bytes()
    assert L.vegas_sparse_decode_attn_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 10 ** 6, FAKE, FAKE, 100000,
                                              FAKE, None, None) == 2
    assert L.vegas_last_error_message().decode() == (
        f"this call needs {need} bytes of scratch, more than the {16 << 20} of the static scratch "
        "(vegas_sparse_decode_attn takes a workspace of any size)")
    # invalid shapes are rejected as by the workspace entry point
    assert L.vegas_sparse_decode_attn_noalloc(ctypes.byref(shape(V, head_dim=96)), FAKE, FAKE, FAKE, FAKE, 100, FAKE,
                                              FAKE, 10, FAKE, None, None) == 2


def test_gather_probe_rejects_bad_arguments(V):
    """The gather-ceiling probe validates its arguments before launching anything."""
    from verification_guided_sparse_verify_amd import build as B
    fn = ctypes.CDLL(B.PROBE_LIB).vegas_probe_gather_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int32] * 8 + [ctypes.c_void_p] * 2

    def call(**kw):
        p = dict(k=FAKE, v=FAKE, rows=FAKE, n=100, total=1000, row=2048, slice=256, heads=8, hpw=2, wgs=256,
                 inflight=2, sink=FAKE)
        p.update(kw)
        return fn(p["k"], p["v"], p["rows"], p["n"], p["total"], p["row"], p["slice"], p["heads"], p["hpw"],
                  p["wgs"], p["inflight"], p["sink"], None)

    assert call(k=None) == -1
    assert call(v=FAKE + 8) == -1              # misaligned
    assert call(n=0) == -1
    assert call(slice=512) == -1               # only 128- or 256-byte slices
    assert call(row=1024) == -1                # eight 256-byte slices do not fit a 1 KB row
    assert call(wgs=258) == -1                 # not a multiple of the four head pairs
    assert call(hpw=3) == -1                   # one or two heads per workgroup
    assert call(heads=7, row=7 * 256) == -1    # an odd head count cannot be paired
    assert call(hpw=1, wgs=260) == -1
    assert call(inflight=4) == -1
    assert call(n=300000, wgs=8) == -1         # more than 4096 entries per workgroup
    assert call(sink=None) == -1


def test_launch_chain_probe_rejects_bad_arguments(V):
    """The dependent-launch probe validates its arguments before launching anything."""
    from verification_guided_sparse_verify_amd import build as B
    fn = ctypes.CDLL(B.PROBE_LIB).vegas_probe_launch_chain
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert fn(10, 256, 0, None, None) == -1         # no sink
    assert fn(0, 256, 0, FAKE, None) == -1          # no launches
    assert fn(100001, 256, 0, FAKE, None) == -1     # too long a chain
    assert fn(10, 0, 0, FAKE, None) == -1           # no workgroups
    assert fn(10, 4097, 0, FAKE, None) == -1
    assert fn(10, 256, -1, FAKE, None) == -1        # LDS outside 0..65536
    assert fn(10, 256, 65537, FAKE, None) == -1
    delay = ctypes.CDLL(B.PROBE_LIB).vegas_probe_delay
    delay.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert delay(1000, None, None) == -1              # no sink
    assert delay(-1, FAKE, None) == -1                # negative
    assert delay(100000001, FAKE, None) == -1         # over a second


def test_trace_build_is_separate_from_the_product_library(V):
    """The phase-timestamp measurement build exports its reader; the product library has no trace
    code (the instrumentation exists only under VEGAS_PHASE_TRACE)."""
    from verification_guided_sparse_verify_amd import build as B
    nm = lambda p: subprocess.run(["nm", "-D", "--defined-only", p], capture_output=True, text=True).stdout
    trace, product = nm(B.TRACE_LIB), nm(V.LIB_PATH)
    assert "vegas_trace_read" in trace and "vegas_trace_set_rotation" in trace
    assert "vegas_trace" not in product
    for name in V.EXPORTED:              # and the same C ABI otherwise
        assert name in trace


def test_verify_select_halves_check_arguments(V):
    """Both halves of the one call validate like it before launching anything."""
    L = V.lib()
    s = shape(V)
    need = V.vegas_verify_select_workspace_size(s, 4, 1000, 4000)
    good = V.host_offsets([0, 1000, 2000, 3000, 4000], [0, 50, 100, 150, 200])
    bad = V.host_offsets([0, 1000, 900, 3000, 4000], [0, 50, 100, 150, 200])
    for name in ("vegas_verify_select_begin_hostplan", "vegas_verify_select_end_hostplan"):
        fn = getattr(L, name)

        def call(host, wsb=need, mask=1 | 16):
            return fn(ctypes.byref(s), 4, FAKE, FAKE, FAKE, FAKE, 1000, 4000, mask, FAKE, FAKE, FAKE, FAKE, FAKE, wsb,
                      None, ctypes.byref(host) if host is not None else None)

        assert call(None) == 1
        assert call(bad) == 1
        assert "decreases" in L.vegas_last_error_message().decode()
        assert call(good, wsb=need - 1) == 3
        assert call(good, mask=0) == 1
