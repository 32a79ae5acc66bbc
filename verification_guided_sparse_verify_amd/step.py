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
                 collect_mask: int | None = None):
        self.inp = inputs
        self.gamma = gamma
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
        self.n_drafts = gamma if n_drafts is None else n_drafts
        self.out = torch.empty_like(q)
        self.scores = torch.empty(num_kv_heads, self.total_kv, dtype=torch.float32, device=dev)
        self.indices = torch.empty(max(self.total_k, 1), dtype=torch.int32, device=dev)
        self.draft_out = torch.empty(max(self.n_drafts, 1), batch, num_q_heads, head_dim, dtype=q.dtype, device=dev)
        ws = max(V.vegas_verify_workspace_size(self.shape, gamma, self.max_seqlen),
                 V.vegas_select_workspace_size(batch, num_kv_heads, gamma, self.max_seqlen, self.total_kv),
                 V.vegas_sparse_decode_workspace_size(self.shape, self.max_k))
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)

    def rebind(self, inputs: dict):
        """Point at another layer's inputs of the same shapes."""
        self.inp = inputs

    def verify(self, collect: bool = True, stream=None):
        i = self.inp
        V.vegas_verify_attn(self.shape, self.gamma, i["q"], i["k"], i["v"], i["cu_seqlens_k"], self.max_seqlen,
                            self.total_kv, self.collect_mask if collect else 0,
                            self.scores if collect else None, self.out, self.workspace, stream)

    def select(self, stream=None):
        i = self.inp
        V.vegas_select_topk(self.batch, self.hkv, self.gamma, self.scores, i["cu_seqlens_k"], self.max_seqlen,
                            self.total_kv, i["cu_k"], self.indices, self.workspace, stream)

    def draft(self, j: int, stream=None):
        i = self.inp
        V.vegas_sparse_decode_attn(self.shape, i["draft_q"][j], i["k"], i["v"], i["cu_seqlens_k"], self.total_kv,
                                   self.indices, i["cu_k"], self.max_k, self.draft_out[j], self.workspace, stream)

    def run(self, stream=None):
        self.verify(True, stream)
        self.select(stream)
        for j in range(self.n_drafts):
            self.draft(j, stream)

    def bind(self, stream=None):
        """Return argument-free callables (verify, verify_plain, select, [draft_j]) with every
        ctypes argument converted once, for launch loops where host time matters."""
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

        common = (shape, self.gamma, i["q"].data_ptr(), i["k"].data_ptr(), i["v"].data_ptr(),
                  i["cu_seqlens_k"].data_ptr(), self.max_seqlen, self.total_kv)
        verify = call(L.vegas_verify_attn, "vegas_verify_attn",
                      common + (self.collect_mask, self.scores.data_ptr(), self.out.data_ptr(), ws, wsb, st))
        plain = call(L.vegas_verify_attn, "vegas_verify_attn",
                     common + (0, None, self.out.data_ptr(), ws, wsb, st))
        select = call(L.vegas_select_topk, "vegas_select_topk",
                      (self.batch, self.hkv, self.gamma, self.scores.data_ptr(), i["cu_seqlens_k"].data_ptr(),
                       self.max_seqlen, self.total_kv, i["cu_k"].data_ptr(), self.indices.data_ptr(), ws, wsb, st))
        drafts = [call(L.vegas_sparse_decode_attn, "vegas_sparse_decode_attn",
                       (shape, i["draft_q"][j].data_ptr(), i["k"].data_ptr(), i["v"].data_ptr(),
                        i["cu_seqlens_k"].data_ptr(), self.total_kv, self.indices.data_ptr(), i["cu_k"].data_ptr(),
                        self.max_k, self.draft_out[j].data_ptr(), ws, wsb, st))
                  for j in range(self.n_drafts)]
        return verify, plain, select, drafts
