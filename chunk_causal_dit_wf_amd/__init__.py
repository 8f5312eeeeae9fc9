"""Chunk-wise causal attention over a rolling paged KV cache, for AMD MI355X (gfx950).

The compute lives in the HIP library ``libwf_chunk_attn.so`` (C ABI in
``include/wf_chunk_attn.h``); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    KVCache, WfError, wf_chunk_attn_fwd, wf_chunk_attn_fwd_noalloc, wf_chunk_attn_plan, wf_chunk_attn_workspace_bytes, workspace_for, wf_kv_append, wf_kv_append_quantize, wf_kv_cache_bytes, wf_kv_cache_check,
    wf_kv_evict, wf_stream_copy, version, lib, LIB_PATH,
    WF_OK, WF_ERR_INVALID_ARG, WF_ERR_UNSUPPORTED, WF_ERR_CAPACITY, WF_ERR_RANGE, WF_ERR_HIP,
    WF_F32, WF_BF16, WF_FP8_E4M3,
)
