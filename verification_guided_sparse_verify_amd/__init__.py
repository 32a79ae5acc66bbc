"""MI355X (gfx950) Vegas attention hot path: verification attention with
Collect-2-Query logit collection, exact top-k KV selection, and sparse
drafting attention over the selected tokens, behind the C ABI of
include/vegas.h.

Importing the package does not load the GPU library; the first call does,
and raises if it has not been built (there is no fallback path).
"""
from .vegas import (  # noqa: F401
    AttnShape, VegasError, attn_shape, lib, status_string,
    vegas_abi_version, vegas_verify_workspace_size, vegas_verify_attn,
    vegas_select_workspace_size, vegas_select_topk,
    vegas_verify_select_workspace_size, vegas_verify_select,
    vegas_sparse_decode_workspace_size, vegas_sparse_decode_attn,
    PagedKV, paged_kv, vegas_verify_paged_workspace_size, vegas_verify_attn_paged,
    vegas_sparse_decode_attn_paged, vegas_verify_local_workspace_size, vegas_verify_attn_local,
    vegas_streaming_indices, vegas_spec_accept_workspace_size, vegas_spec_accept,
    VEGAS_DTYPE_F32, VEGAS_DTYPE_BF16,
)
