"""Python access to the plain CPU oracle of the Vegas attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library and
its Python binding never import it; the two share no code.

The arithmetic lives in ``vegas_oracle.c`` (IEEE double throughout).  This
module only builds that file with gcc, loads it with ctypes and marshals numpy
arrays.  Inputs are passed as the exact element bits the GPU reads: float32
arrays for fp32 data, uint16 arrays holding bf16 bit patterns for bf16 data.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vegas_oracle.c")
_SO = os.path.join(_HERE, "libvegas_oracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

_lib_handle = None


def build() -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) and return the .so path."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        D = ctypes.c_double
        U32 = ctypes.c_uint32
        lib.vo_verify_attn.argtypes = [I, I, I, I, I, I, D, P, P, P, P, I64, U32, P, P]
        lib.vo_verify_attn.restype = I
        lib.vo_verify_attn_local.argtypes = [I, I, I, I, I, I, D, P, P, P, P, I64, I, U32, P, P]
        lib.vo_verify_attn_local.restype = I
        lib.vo_streaming_indices.argtypes = [I, I, I, P, P, P]
        lib.vo_streaming_indices.restype = I
        lib.vo_spec_accept.argtypes = [I, I, I64, P, P, P, P, P, P, P]
        lib.vo_spec_accept.restype = I
        lib.vo_select_topk.argtypes = [I, I, I, P, P, I64, P, P, P, P]
        lib.vo_select_topk.restype = I
        lib.vo_sparse_decode_attn.argtypes = [I, I, I, I, I, D, P, P, P, P, P, P, P]
        lib.vo_sparse_decode_attn.restype = I
        _lib_handle = lib
    return _lib_handle


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def verify_attn(q, k, v, cu_seqlens_k, gamma: int, scale: float,
                collect_mask: int | None = None, want_scores: bool = True, window: int = 0):
    """Verification attention over the gamma+1 new rows of each sequence.

    q: [batch*(gamma+1), Hq, D]; k, v: [total_kv, Hkv, D]; cu_seqlens_k: [batch+1].
    collect_mask defaults to the Collect-2-Query rows {0, gamma}.  window > 0 applies a local
    mask (row r sees the `window` newest keys up to its position) and needs want_scores=False.
    Returns (out float64 [batch*(gamma+1), Hq, D], scores float64 [Hkv, total_kv] or None).
    """
    q, k, v = _c(q), _c(k), _c(v)
    cu = _c(cu_seqlens_k, np.int32)
    code = _dtype_code(q)
    assert _dtype_code(k) == code and _dtype_code(v) == code
    batch = cu.shape[0] - 1
    _, hq, d = q.shape
    total, hkv, d2 = k.shape
    assert d == d2 and v.shape == k.shape and q.shape[0] == batch * (gamma + 1)
    if collect_mask is None:
        collect_mask = (1 | (1 << gamma))
    out = np.zeros(q.shape, dtype=np.float64)
    scores = np.zeros((hkv, total), dtype=np.float64) if want_scores else None
    rc = _lib().vo_verify_attn_local(code, batch, hq, hkv, d, gamma, float(scale),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(cu), total, int(window),
                                     collect_mask & 0xFFFFFFFF, _ptr(out), _ptr(scores))
    if rc != 0:
        raise ValueError("vo_verify_attn rejected its arguments")
    return out, scores


def select_topk(scores, cu_seqlens_k, gamma: int, cu_k):
    """Exact per-sequence top-k of the KV-head-summed score.

    Returns (indices int32 [cu_k[-1]], theta float64 [batch], S float64 [total_kv]).
    """
    scores = _c(scores, np.float64)
    cu = _c(cu_seqlens_k, np.int32)
    cuk = _c(cu_k, np.int32)
    batch = cu.shape[0] - 1
    hkv, total = scores.shape
    indices = np.zeros(max(int(cuk[-1]), 1), dtype=np.int32)
    theta = np.zeros(batch, dtype=np.float64)
    S = np.zeros(total, dtype=np.float64)
    rc = _lib().vo_select_topk(batch, hkv, gamma, _ptr(scores), _ptr(cu), total,
                               _ptr(cuk), _ptr(indices), _ptr(theta), _ptr(S))
    if rc != 0:
        raise ValueError("vo_select_topk rejected its arguments")
    return indices[: int(cuk[-1])], theta, S


def sparse_decode_attn(q, k, v, cu_seqlens_k, indices, cu_idx, scale: float):
    """Single-query attention per head over per-sequence index lists.

    q: [batch, Hq, D]; indices relative to each sequence start.  Returns float64 [batch, Hq, D].
    """
    q, k, v = _c(q), _c(k), _c(v)
    cu = _c(cu_seqlens_k, np.int32)
    idx = _c(indices, np.int32)
    if idx.size == 0:
        idx = np.zeros(1, dtype=np.int32)
    cui = _c(cu_idx, np.int32)
    code = _dtype_code(q)
    batch = cu.shape[0] - 1
    _, hq, d = q.shape
    _, hkv, _ = k.shape
    out = np.zeros(q.shape, dtype=np.float64)
    rc = _lib().vo_sparse_decode_attn(code, batch, hq, hkv, d, float(scale), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(cu), _ptr(idx), _ptr(cui), _ptr(out))
    if rc != 0:
        raise ValueError("vo_sparse_decode_attn rejected its arguments")
    return out


def streaming_indices(cu_seqlens_k, gamma: int, sinks: int, cu_idx):
    """Sink-plus-recent lists with per-sequence budgets cu_idx; returns int32 [cu_idx[-1]]."""
    cu = _c(cu_seqlens_k, np.int32)
    cui = _c(cu_idx, np.int32)
    out = np.zeros(max(int(cui[-1]), 1), dtype=np.int32)
    rc = _lib().vo_streaming_indices(cu.shape[0] - 1, gamma, sinks, _ptr(cu), _ptr(cui), _ptr(out))
    if rc != 0:
        raise ValueError("vo_streaming_indices rejected its arguments")
    return out[: int(cui[-1])]


def spec_accept(p, q, draft, u_accept, u_sample):
    """Speculative-sampling acceptance.  p: float32 [B, gamma+1, V]; q: float32 [B, gamma, V];
    draft: int32 [B, gamma]; u_accept: float32 [B, gamma]; u_sample: float32 [B].
    Returns (n_accepted int32 [B], next_token int32 [B])."""
    p = _c(p, np.float32)
    B, W, V = p.shape
    gamma = W - 1
    q = _c(q, np.float32) if gamma > 0 else None
    draft = _c(draft, np.int32) if gamma > 0 else None
    ua = _c(u_accept, np.float32) if gamma > 0 else None
    us = _c(u_sample, np.float32)
    n = np.zeros(B, np.int32)
    t = np.zeros(B, np.int32)
    rc = _lib().vo_spec_accept(B, gamma, V, _ptr(p), _ptr(q), _ptr(draft), _ptr(ua), _ptr(us), _ptr(n), _ptr(t))
    if rc != 0:
        raise ValueError("vo_spec_accept rejected its arguments")
    return n, t
