"""One Vegas layer-step on device buffers: verify (with Collect-2-Query),
select, then gamma sparse drafts over the selected positions.

Orchestration only: buffers come from torch, every computation is a call into
libvegas.so on one HIP stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import vegas as V


class LayerStep:
    """Holds the output buffers and workspaces of one layer's step.

    inputs: dict with q [B*W, Hq, D], k, v [total_kv, Hkv, D], cu_seqlens_k,
    cu_k (int32 [B+1], device) and draft_q [n_drafts, B, Hq, D].
    """

    def __init__(self, inputs: dict, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 gamma: int, seqlens, k_per_seq, softmax_scale: float, n_drafts: int | None = None,
                 collect_mask: int | None = None, paged: dict | None = None, selection: str = "vegas",
                 sinks: int = 4):
        self.inp = inputs
        self.gamma = gamma
        # selection: "vegas" (verification-guided top-k of the collected logits) or "streaming"
        # (query-agnostic sinks + most recent tokens with the same budget; no collection).
        assert selection in ("vegas", "streaming")
        self.selection = selection
        self.sinks = sinks
        # paged: a page pool from workloads.page_cache (k_pool, v_pool, block_table, num_pages); the
        # paged entry points then read K/V through the block table.
        self.paged = paged
        self.page_size = paged["k_pool"].shape[1] if paged else 0
        self.pages = V.paged_kv(paged["block_table"], self.page_size, paged["num_pages"]) if paged else None
        q = inputs["q"]
        dev = q.device
        dtype = V.VEGAS_DTYPE_BF16 if q.dtype == torch.bfloat16 else V.VEGAS_DTYPE_F32
        self.shape = V.attn_shape(dtype, batch, num_q_heads, num_kv_heads, head_dim, softmax_scale)
        self.batch, self.hq, self.hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.max_seqlen = int(max(seqlens))
        self.total_kv = int(sum(seqlens))
        self.max_k = int(max(k_per_seq)) if len(k_per_seq) else 0
        self.total_k = int(sum(k_per_seq))
        self.collect_mask = (1 | (1 << gamma)) if collect_mask is None else collect_mask
        # host copies of cu_seqlens_k and cu_k, for the host-planned entry points
        cu, cuk = [0], [0]
        for n, kk in zip(seqlens, k_per_seq):
            cu.append(cu[-1] + int(n))
            cuk.append(cuk[-1] + int(kk))
        self.host = V.host_offsets(cu, cuk)
        self.n_drafts = gamma if n_drafts is None else n_drafts
        self.out = torch.empty_like(q)
        self.scores = torch.empty(num_kv_heads, self.total_kv, dtype=torch.float32, device=dev)
        self.indices = torch.empty(max(self.total_k, 1), dtype=torch.int32, device=dev)
        self.draft_out = torch.empty(max(self.n_drafts, 1), batch, num_q_heads, head_dim, dtype=q.dtype, device=dev)
        ws = max(V.vegas_verify_paged_workspace_size(self.shape, gamma, self.max_seqlen, self.page_size),
                 V.vegas_select_workspace_size(batch, num_kv_heads, gamma, self.max_seqlen, self.total_kv),
                 V.vegas_sparse_decode_workspace_size(self.shape, self.max_k))
        if self.fusable:
            ws = max(ws, V.vegas_verify_select_workspace_size(self.shape, gamma, self.max_seqlen, self.total_kv))
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)

    def rebind(self, inputs: dict):
        """Point at another layer's inputs of the same shapes."""
        self.inp = inputs

    def verify(self, collect: bool = True, stream=None, host_plan: bool = False):
        i = self.inp
        mask, scores = (self.collect_mask, self.scores) if collect else (0, None)
        if host_plan and not self.paged:
            V.vegas_verify_attn_hostplan(self.shape, self.gamma, i["q"], i["k"], i["v"], i["cu_seqlens_k"],
                                         self.max_seqlen, self.total_kv, mask, scores, self.out, self.workspace,
                                         self.host, stream)
            return
        if self.paged:
            V.vegas_verify_attn_paged(self.shape, self.gamma, i["q"], self.paged["k_pool"], self.paged["v_pool"],
                                      self.pages, i["cu_seqlens_k"], self.max_seqlen, self.total_kv, mask, scores,
                                      self.out, self.workspace, stream)
            return
        V.vegas_verify_attn(self.shape, self.gamma, i["q"], i["k"], i["v"], i["cu_seqlens_k"], self.max_seqlen,
                            self.total_kv, mask, scores, self.out, self.workspace, stream)

    @property
    def fusable(self) -> bool:
        """Verification and selection can run as one call (contiguous cache, Vegas selection)."""
        return not self.paged and self.selection == "vegas"

    def verify_select(self, stream=None, host_plan: bool = False):
        """Verification with collection followed by selection, as one library call (host_plan: the
        call that also takes host copies of the offsets)."""
        i = self.inp
        if host_plan:
            V.vegas_verify_select_hostplan(self.shape, self.gamma, i["q"], i["k"], i["v"], i["cu_seqlens_k"],
                                           self.max_seqlen, self.total_kv, self.collect_mask, i["cu_k"], self.scores,
                                           self.indices, self.out, self.workspace, self.host, stream)
            return
        V.vegas_verify_select(self.shape, self.gamma, i["q"], i["k"], i["v"], i["cu_seqlens_k"], self.max_seqlen,
                              self.total_kv, self.collect_mask, i["cu_k"], self.scores, self.indices, self.out,
                              self.workspace, stream)

    def select(self, stream=None):
        i = self.inp
        if self.selection == "streaming":
            V.vegas_streaming_indices(self.batch, self.gamma, self.sinks, i["cu_seqlens_k"], self.total_kv, i["cu_k"],
                                      self.total_k, self.indices, stream)
            return
        V.vegas_select_topk(self.batch, self.hkv, self.gamma, self.scores, i["cu_seqlens_k"], self.max_seqlen,
                            self.total_kv, i["cu_k"], self.indices, self.workspace, stream)

    def draft(self, j: int, stream=None, host_plan: bool = False):
        i = self.inp
        if host_plan and not self.paged:
            V.vegas_sparse_decode_attn_hostplan(self.shape, i["draft_q"][j], i["k"], i["v"], i["cu_seqlens_k"],
                                                self.total_kv, self.indices, i["cu_k"], self.max_k, self.draft_out[j],
                                                self.workspace, self.host, stream)
            return
        if self.paged:
            V.vegas_sparse_decode_attn_paged(self.shape, i["draft_q"][j], self.paged["k_pool"], self.paged["v_pool"],
                                             self.pages, i["cu_seqlens_k"], self.total_kv, self.indices, i["cu_k"],
                                             self.max_k, self.draft_out[j], self.workspace, stream)
            return
        V.vegas_sparse_decode_attn(self.shape, i["draft_q"][j], i["k"], i["v"], i["cu_seqlens_k"], self.total_kv,
                                   self.indices, i["cu_k"], self.max_k, self.draft_out[j], self.workspace, stream)

    def run(self, stream=None, fused: bool = False, host_plan: bool = False, select_stream=None):
        """One layer step.  select_stream (with fused and host_plan): the selection's last steps run
        there after the verification kernels, and the drafting passes wait for them."""
        if fused and select_stream is not None:
            launch = stream if stream is not None else torch.cuda.current_stream()
            self.bind_fused(launch, part="begin")()
            verified = torch.cuda.Event()
            verified.record(launch)
            select_stream.wait_event(verified)
            self.bind_fused(select_stream, part="end")()
            selected = torch.cuda.Event()
            selected.record(select_stream)
            launch.wait_event(selected)
        elif fused:
            self.verify_select(stream, host_plan)
        else:
            self.verify(self.selection == "vegas", stream)
            self.select(stream)
        for j in range(self.n_drafts):
            self.draft(j, stream, host_plan)

    def bind(self, stream=None, host_plan: bool = False):
        """Return argument-free callables (verify, verify_plain, select, [draft_j]) with every
        ctypes argument converted once, for launch loops where host time matters (host_plan:
        verification and drafting go through the host-planned entry points)."""
        i = self.inp
        st = V._stream(stream)
        shape = ctypes.byref(self.shape)
        ws, wsb = self.workspace.data_ptr(), self.workspace.numel()
        L = V.lib()

        def call(fn, name, args):
            def go():
                rc = fn(*args)
                if rc:
                    V._check(rc, name)
            return go

        if self.paged:
            kp, vp = self.paged["k_pool"].data_ptr(), self.paged["v_pool"].data_ptr()
            pages = ctypes.byref(self.pages)
            vfn, vname = L.vegas_verify_attn_paged, "vegas_verify_attn_paged"
            common = (shape, self.gamma, i["q"].data_ptr(), kp, vp, pages, i["cu_seqlens_k"].data_ptr(),
                      self.max_seqlen, self.total_kv)
            dfn, dname = L.vegas_sparse_decode_attn_paged, "vegas_sparse_decode_attn_paged"
            kv = (kp, vp, pages)
        else:
            vfn, vname = L.vegas_verify_attn, "vegas_verify_attn"
            common = (shape, self.gamma, i["q"].data_ptr(), i["k"].data_ptr(), i["v"].data_ptr(),
                      i["cu_seqlens_k"].data_ptr(), self.max_seqlen, self.total_kv)
            dfn, dname = L.vegas_sparse_decode_attn, "vegas_sparse_decode_attn"
            kv = (i["k"].data_ptr(), i["v"].data_ptr())
        vtail = ()
        if host_plan and not self.paged:
            vfn, vname = L.vegas_verify_attn_hostplan, "vegas_verify_attn_hostplan"
            vtail = (ctypes.byref(self.host),)
        verify = call(vfn, vname,
                      common + (self.collect_mask, self.scores.data_ptr(), self.out.data_ptr(), ws, wsb, st) + vtail)
        plain = call(vfn, vname, common + (0, None, self.out.data_ptr(), ws, wsb, st) + vtail)
        if self.selection == "streaming":
            select = call(L.vegas_streaming_indices, "vegas_streaming_indices",
                          (self.batch, self.gamma, self.sinks, i["cu_seqlens_k"].data_ptr(), self.total_kv,
                           i["cu_k"].data_ptr(), self.total_k, self.indices.data_ptr(), st))
            verify = plain          # nothing is collected for a query-agnostic selection
        else:
            select = call(L.vegas_select_topk, "vegas_select_topk",
                          (self.batch, self.hkv, self.gamma, self.scores.data_ptr(), i["cu_seqlens_k"].data_ptr(),
                           self.max_seqlen, self.total_kv, i["cu_k"].data_ptr(), self.indices.data_ptr(), ws, wsb,
                           st))
        tail = ()
        if host_plan and not self.paged:
            dfn, dname = L.vegas_sparse_decode_attn_hostplan, "vegas_sparse_decode_attn_hostplan"
            tail = (ctypes.byref(self.host),)
        drafts = [call(dfn, dname,
                       (shape, i["draft_q"][j].data_ptr()) + kv +
                       (i["cu_seqlens_k"].data_ptr(), self.total_kv, self.indices.data_ptr(), i["cu_k"].data_ptr(),
                        self.max_k, self.draft_out[j].data_ptr(), ws, wsb, st) + tail)
                  for j in range(self.n_drafts)]
        return verify, plain, select, drafts

    def bind_fused(self, stream=None, host_plan: bool = False, part: str = ""):
        """Argument-free callable of the one-call verification + selection (host_plan: the
        host-planned entry point; part "begin" or "end": that half of it, host-planned)."""
        if not self.fusable:
            raise ValueError("the one-call verification + selection needs a contiguous cache and Vegas selection")
        i = self.inp
        args = (ctypes.byref(self.shape), self.gamma, i["q"].data_ptr(), i["k"].data_ptr(), i["v"].data_ptr(),
                i["cu_seqlens_k"].data_ptr(), self.max_seqlen, self.total_kv, self.collect_mask,
                i["cu_k"].data_ptr(), self.scores.data_ptr(), self.indices.data_ptr(), self.out.data_ptr(),
                self.workspace.data_ptr(), self.workspace.numel(), V._stream(stream))
        name = "vegas_verify_select"
        if host_plan or part:
            args += (ctypes.byref(self.host),)
            name = f"vegas_verify_select_{part}_hostplan" if part else "vegas_verify_select_hostplan"
        fn = getattr(V.lib(), name)

        def go():
            rc = fn(*args)
            if rc:
                V._check(rc, name)
        return go
