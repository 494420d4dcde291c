"""Selected-KV paged decode attention on MI355X (gfx950): Python binding.

Thin ctypes wrappers over libkap.so (include/kap.h) with the same names as the
C entry points.  They only marshal arguments: every step of the path runs in
the library's HIP kernels.  PyTorch supplies device memory and the current
stream.  If libkap.so has not been built the first call raises
KapLibraryMissing -- there is no fallback of any kind.

Tensor conventions: bf16 data may be torch.bfloat16 or 16-bit integer tensors
holding bf16 bit patterns; fp32 data are torch.float32; index tensors int32
(slot mapping int64).  All tensors must be contiguous and on the same GPU.
"""
from ._lib import (  # noqa: F401
    BF16, F32, PLAN_FULL_BOUNDARY, PLAN_FULL_CAPACITY, PLAN_FULL_MARGIN, PLAN_SELECTED, KapError,
    KapLibraryMissing, alloc_kv_pools, append_kv, attn_workspace_bytes, budget_from_ratio,
    choose_plan, build_summary, compact_view, copy_kv_pools, decode_attn, decode_attn_noalloc,
    diag_stream_read, host_proxy_query, host_score_blocks, host_select_topk, kv_pool_layout,
    lib_path, load, materialize_view, proxy_pack_weights, proxy_query, proxy_query_packed,
    proxy_workspace_bytes, score_blocks, score_pool_blocks, select_compact, select_topk,
    update_summary, verify_attn, version,
)
from .tags import format_split_tag, middle_count, parse_split_tag  # noqa: F401,E402
