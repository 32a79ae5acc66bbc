"""Thin ctypes binding of libvegas.so (include/vegas.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of the library.  Tensor arguments are torch tensors that already live
on the GPU (torch supplies device memory and streams); they are passed as raw
device pointers.  If the library has not been built, every call raises -- there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvegas.so")

VEGAS_OK = 0
VEGAS_ERR_INVALID_ARGUMENT = 1
VEGAS_ERR_UNSUPPORTED = 2
VEGAS_ERR_WORKSPACE_TOO_SMALL = 3
VEGAS_ERR_HIP = 4

VEGAS_DTYPE_F32 = 0
VEGAS_DTYPE_BF16 = 1

EXPORTED = (
    "vegas_abi_version", "vegas_status_string", "vegas_last_error_message",
    "vegas_verify_workspace_size", "vegas_verify_attn",
    "vegas_select_workspace_size", "vegas_select_topk",
    "vegas_verify_select_workspace_size", "vegas_verify_select",
    "vegas_sparse_decode_workspace_size", "vegas_sparse_decode_attn",
    "vegas_verify_paged_workspace_size", "vegas_verify_attn_paged", "vegas_sparse_decode_attn_paged",
    "vegas_verify_local_workspace_size", "vegas_verify_attn_local", "vegas_streaming_indices",
    "vegas_spec_accept_workspace_size", "vegas_spec_accept",
    "vegas_verify_attn_hostplan", "vegas_verify_select_hostplan", "vegas_sparse_decode_attn_hostplan",
    "vegas_verify_hostplan_info", "vegas_sparse_decode_attn_noalloc", "vegas_noalloc_scratch_bytes",
    "vegas_verify_select_begin_hostplan", "vegas_verify_select_end_hostplan",
)


class VegasError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn} -> {status_string(status)}: {detail}")


class AttnShape(ctypes.Structure):
    """vegas_attn_shape_t."""
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class PagedKV(ctypes.Structure):
    """vegas_paged_kv_t."""
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class HostOffsets(ctypes.Structure):
    """vegas_host_offsets_t: host copies of cu_seqlens_k and of cu_k / cu_idx."""
    _fields_ = [("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32)), ("cu_idx", ctypes.POINTER(ctypes.c_int32))]


def host_offsets(cu_seqlens_k, cu_idx) -> HostOffsets:
    """Host offsets from two integer sequences (lists, numpy arrays or CPU tensors); the
    returned structure owns copies of both."""
    a = (ctypes.c_int32 * len(cu_seqlens_k))(*[int(x) for x in cu_seqlens_k])
    b = (ctypes.c_int32 * len(cu_idx))(*[int(x) for x in cu_idx])
    h = HostOffsets(ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)), ctypes.cast(b, ctypes.POINTER(ctypes.c_int32)))
    h._keep = (a, b)
    return h


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        SP = ctypes.POINTER(AttnShape)
        PP = ctypes.POINTER(PagedKV)
        PSZ = ctypes.POINTER(ctypes.c_size_t)
        HP = ctypes.POINTER(HostOffsets)
        sig = {
            "vegas_abi_version": ([], I32),
            "vegas_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "vegas_last_error_message": ([], ctypes.c_char_p),
            "vegas_verify_workspace_size": ([SP, I32, I32, PSZ], ctypes.c_int),
            "vegas_verify_attn": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, SZ, P], ctypes.c_int),
            "vegas_select_workspace_size": ([I32, I32, I32, I32, I32, PSZ], ctypes.c_int),
            "vegas_select_topk": ([I32, I32, I32, P, P, I32, I32, P, P, P, SZ, P], ctypes.c_int),
            "vegas_verify_select_workspace_size": ([SP, I32, I32, I32, PSZ], ctypes.c_int),
            "vegas_verify_select": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, P, P, SZ, P], ctypes.c_int),
            "vegas_sparse_decode_workspace_size": ([SP, I32, PSZ], ctypes.c_int),
            "vegas_sparse_decode_attn": ([SP, P, P, P, P, I32, P, P, I32, P, P, SZ, P], ctypes.c_int),
            "vegas_verify_paged_workspace_size": ([SP, I32, I32, I32, PSZ], ctypes.c_int),
            "vegas_verify_attn_paged": ([SP, I32, P, P, P, PP, P, I32, I32, U32, P, P, P, SZ, P], ctypes.c_int),
            "vegas_sparse_decode_attn_paged": ([SP, P, P, P, PP, P, I32, P, P, I32, P, P, SZ, P], ctypes.c_int),
            "vegas_verify_local_workspace_size": ([SP, I32, I32, I32, PSZ], ctypes.c_int),
            "vegas_verify_attn_local": ([SP, I32, P, P, P, P, I32, I32, I32, P, P, SZ, P], ctypes.c_int),
            "vegas_streaming_indices": ([I32, I32, I32, P, I32, P, I32, P, P], ctypes.c_int),
            "vegas_spec_accept_workspace_size": ([I32, I32, PSZ], ctypes.c_int),
            "vegas_spec_accept": ([I32, I32, I32, P, P, P, P, P, P, P, P, SZ, P], ctypes.c_int),
            "vegas_verify_attn_hostplan": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, SZ, P, HP], ctypes.c_int),
            "vegas_verify_select_hostplan": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, P, P, SZ, P, HP],
                                             ctypes.c_int),
            "vegas_sparse_decode_attn_hostplan": ([SP, P, P, P, P, I32, P, P, I32, P, P, SZ, P, HP], ctypes.c_int),
            "vegas_verify_hostplan_info": ([SP, I32, I32, I32, HP, ctypes.POINTER(I32), ctypes.POINTER(I32)],
                                           ctypes.c_int),
            "vegas_sparse_decode_attn_noalloc": ([SP, P, P, P, P, I32, P, P, I32, P, P, HP], ctypes.c_int),
            "vegas_noalloc_scratch_bytes": ([], SZ),
            "vegas_verify_select_begin_hostplan": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, P, P, SZ, P, HP],
                                                   ctypes.c_int),
            "vegas_verify_select_end_hostplan": ([SP, I32, P, P, P, P, I32, I32, U32, P, P, P, P, P, SZ, P, HP],
                                                 ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().vegas_status_string(status).decode()


def _check(status: int, fn: str):
    if status != VEGAS_OK:
        raise VegasError(status, fn, lib().vegas_last_error_message().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def attn_shape(dtype: int, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
               softmax_scale: float) -> AttnShape:
    return AttnShape(dtype, batch, num_q_heads, num_kv_heads, head_dim, softmax_scale)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def vegas_abi_version() -> int:
    return lib().vegas_abi_version()


def vegas_verify_workspace_size(shape: AttnShape, gamma: int, max_seqlen_k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_verify_workspace_size(ctypes.byref(shape), gamma, max_seqlen_k, ctypes.byref(n)),
           "vegas_verify_workspace_size")
    return n.value


def vegas_verify_attn(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int,
                      total_kv: int, collect_mask: int, scores, out, workspace, stream=None) -> None:
    _check(lib().vegas_verify_attn(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(cu_seqlens_k), max_seqlen_k, total_kv, collect_mask & 0xFFFFFFFF,
                                   _ptr(scores), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)),
           "vegas_verify_attn")


def vegas_select_workspace_size(batch: int, num_kv_heads: int, gamma: int, max_seqlen_k: int,
                                total_kv: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_select_workspace_size(batch, num_kv_heads, gamma, max_seqlen_k, total_kv,
                                             ctypes.byref(n)),
           "vegas_select_workspace_size")
    return n.value


def vegas_select_topk(batch: int, num_kv_heads: int, gamma: int, scores, cu_seqlens_k, max_seqlen_k: int,
                      total_kv: int, cu_k, indices, workspace, stream=None) -> None:
    _check(lib().vegas_select_topk(batch, num_kv_heads, gamma, _ptr(scores), _ptr(cu_seqlens_k), max_seqlen_k,
                                   total_kv, _ptr(cu_k), _ptr(indices), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)),
           "vegas_select_topk")


def vegas_verify_select_workspace_size(shape: AttnShape, gamma: int, max_seqlen_k: int, total_kv: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_verify_select_workspace_size(ctypes.byref(shape), gamma, max_seqlen_k, total_kv,
                                                    ctypes.byref(n)),
           "vegas_verify_select_workspace_size")
    return n.value


def vegas_verify_select(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int, total_kv: int,
                        collect_mask: int, cu_k, scores, indices, out, workspace, stream=None) -> None:
    _check(lib().vegas_verify_select(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k),
                                     max_seqlen_k, total_kv, collect_mask & 0xFFFFFFFF, _ptr(cu_k), _ptr(scores),
                                     _ptr(indices), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                     _stream(stream)),
           "vegas_verify_select")


def vegas_verify_attn_hostplan(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int,
                               total_kv: int, collect_mask: int, scores, out, workspace, host: HostOffsets,
                               stream=None) -> None:
    _check(lib().vegas_verify_attn_hostplan(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(cu_seqlens_k), max_seqlen_k, total_kv, collect_mask & 0xFFFFFFFF,
                                            _ptr(scores), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                            _stream(stream), ctypes.byref(host)),
           "vegas_verify_attn_hostplan")


def vegas_sparse_decode_attn_noalloc(shape: AttnShape, q, k, v, cu_seqlens_k, total_kv: int, indices, cu_idx,
                                     max_idx: int, out, stream=None, host: HostOffsets | None = None) -> None:
    """vegas_sparse_decode_attn on the library's static scratch (no workspace argument)."""
    _check(lib().vegas_sparse_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k),
                                                  total_kv, _ptr(indices), _ptr(cu_idx), max_idx, _ptr(out),
                                                  _stream(stream), ctypes.byref(host) if host is not None else None),
           "vegas_sparse_decode_attn_noalloc")


def vegas_noalloc_scratch_bytes() -> int:
    return int(lib().vegas_noalloc_scratch_bytes())


def vegas_verify_hostplan_info(shape: AttnShape, gamma: int, max_seqlen_k: int, total_kv: int,
                               host: HostOffsets) -> tuple[bool, int]:
    """(balanced, workgroups per KV head) of the split plan a host-planned verification takes."""
    bal, wgs = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().vegas_verify_hostplan_info(ctypes.byref(shape), gamma, max_seqlen_k, total_kv, ctypes.byref(host),
                                            ctypes.byref(bal), ctypes.byref(wgs)),
           "vegas_verify_hostplan_info")
    return bool(bal.value), int(wgs.value)


def vegas_verify_select_hostplan(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int,
                                 total_kv: int, collect_mask: int, cu_k, scores, indices, out, workspace,
                                 host: HostOffsets, stream=None) -> None:
    _check(lib().vegas_verify_select_hostplan(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(cu_seqlens_k), max_seqlen_k, total_kv, collect_mask & 0xFFFFFFFF,
                                              _ptr(cu_k), _ptr(scores), _ptr(indices), _ptr(out), _ptr(workspace),
                                              _nbytes(workspace), _stream(stream), ctypes.byref(host)),
           "vegas_verify_select_hostplan")


def _verify_select_half(name, shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k, total_kv, collect_mask, cu_k, scores,
                        indices, out, workspace, host, stream):
    _check(getattr(lib(), name)(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), max_seqlen_k,
                                total_kv, collect_mask & 0xFFFFFFFF, _ptr(cu_k), _ptr(scores), _ptr(indices), _ptr(out),
                                _ptr(workspace), _nbytes(workspace), _stream(stream), ctypes.byref(host)), name)


def vegas_verify_select_begin_hostplan(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int,
                                       total_kv: int, collect_mask: int, cu_k, scores, indices, out, workspace,
                                       host: HostOffsets, stream=None) -> None:
    _verify_select_half("vegas_verify_select_begin_hostplan", shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k,
                        total_kv, collect_mask, cu_k, scores, indices, out, workspace, host, stream)


def vegas_verify_select_end_hostplan(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int,
                                     total_kv: int, collect_mask: int, cu_k, scores, indices, out, workspace,
                                     host: HostOffsets, stream=None) -> None:
    _verify_select_half("vegas_verify_select_end_hostplan", shape, gamma, q, k, v, cu_seqlens_k, max_seqlen_k,
                        total_kv, collect_mask, cu_k, scores, indices, out, workspace, host, stream)


def vegas_sparse_decode_workspace_size(shape: AttnShape, max_idx: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_sparse_decode_workspace_size(ctypes.byref(shape), max_idx, ctypes.byref(n)),
           "vegas_sparse_decode_workspace_size")
    return n.value


def vegas_sparse_decode_attn(shape: AttnShape, q, k, v, cu_seqlens_k, total_kv: int, indices, cu_idx,
                             max_idx: int, out, workspace, stream=None) -> None:
    _check(lib().vegas_sparse_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k),
                                          total_kv, _ptr(indices), _ptr(cu_idx), max_idx, _ptr(out),
                                          _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "vegas_sparse_decode_attn")


def vegas_sparse_decode_attn_hostplan(shape: AttnShape, q, k, v, cu_seqlens_k, total_kv: int, indices, cu_idx,
                                      max_idx: int, out, workspace, host: HostOffsets, stream=None) -> None:
    _check(lib().vegas_sparse_decode_attn_hostplan(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(cu_seqlens_k), total_kv, _ptr(indices), _ptr(cu_idx),
                                                   max_idx, _ptr(out), _ptr(workspace), _nbytes(workspace),
                                                   _stream(stream), ctypes.byref(host)),
           "vegas_sparse_decode_attn_hostplan")


def paged_kv(block_table, page_size: int, num_pages: int) -> PagedKV:
    """block_table: device int32 tensor [batch, max_pages_per_seq]."""
    return PagedKV(_ptr(block_table), block_table.shape[1], page_size, num_pages)


def vegas_verify_paged_workspace_size(shape: AttnShape, gamma: int, max_seqlen_k: int, page_size: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_verify_paged_workspace_size(ctypes.byref(shape), gamma, max_seqlen_k, page_size,
                                                   ctypes.byref(n)),
           "vegas_verify_paged_workspace_size")
    return n.value


def vegas_verify_attn_paged(shape: AttnShape, gamma: int, q, k, v, pages: PagedKV, cu_seqlens_k,
                            max_seqlen_k: int, total_kv: int, collect_mask: int, scores, out, workspace,
                            stream=None) -> None:
    _check(lib().vegas_verify_attn_paged(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(pages),
                                         _ptr(cu_seqlens_k), max_seqlen_k, total_kv, collect_mask & 0xFFFFFFFF,
                                         _ptr(scores), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                         _stream(stream)),
           "vegas_verify_attn_paged")


def vegas_sparse_decode_attn_paged(shape: AttnShape, q, k, v, pages: PagedKV, cu_seqlens_k, total_kv: int, indices,
                                   cu_idx, max_idx: int, out, workspace, stream=None) -> None:
    _check(lib().vegas_sparse_decode_attn_paged(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(pages),
                                                _ptr(cu_seqlens_k), total_kv, _ptr(indices), _ptr(cu_idx), max_idx,
                                                _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "vegas_sparse_decode_attn_paged")


def vegas_verify_local_workspace_size(shape: AttnShape, gamma: int, max_seqlen_k: int, window: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_verify_local_workspace_size(ctypes.byref(shape), gamma, max_seqlen_k, window,
                                                   ctypes.byref(n)),
           "vegas_verify_local_workspace_size")
    return n.value


def vegas_verify_attn_local(shape: AttnShape, gamma: int, q, k, v, cu_seqlens_k, max_seqlen_k: int, total_kv: int,
                            window: int, out, workspace, stream=None) -> None:
    _check(lib().vegas_verify_attn_local(ctypes.byref(shape), gamma, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_k),
                                         max_seqlen_k, total_kv, window, _ptr(out), _ptr(workspace),
                                         _nbytes(workspace), _stream(stream)),
           "vegas_verify_attn_local")


def vegas_streaming_indices(batch: int, gamma: int, sinks: int, cu_seqlens_k, total_kv: int, cu_idx, total_idx: int,
                            indices, stream=None) -> None:
    _check(lib().vegas_streaming_indices(batch, gamma, sinks, _ptr(cu_seqlens_k), total_kv, _ptr(cu_idx), total_idx,
                                         _ptr(indices), _stream(stream)),
           "vegas_streaming_indices")


def vegas_spec_accept_workspace_size(batch: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vegas_spec_accept_workspace_size(batch, vocab, ctypes.byref(n)), "vegas_spec_accept_workspace_size")
    return n.value


def vegas_spec_accept(batch: int, gamma: int, vocab: int, p, q, draft_tokens, u_accept, u_sample, n_accepted,
                      next_token, workspace=None, stream=None) -> None:
    """workspace: a device uint8 tensor of vegas_spec_accept_workspace_size bytes (allocated here if None)."""
    if workspace is None:
        import torch
        workspace = torch.empty(vegas_spec_accept_workspace_size(batch, vocab), dtype=torch.uint8, device=p.device)
    _check(lib().vegas_spec_accept(batch, gamma, vocab, _ptr(p), _ptr(q), _ptr(draft_tokens), _ptr(u_accept),
                                   _ptr(u_sample), _ptr(n_accepted), _ptr(next_token), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream)),
           "vegas_spec_accept")
