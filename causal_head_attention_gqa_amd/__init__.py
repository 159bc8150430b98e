"""MI355X (gfx950) causal attention: prefill, chunked prefill against a KV cache, KV-cache append,
KV-cache decode (GQA and MLA-absorbed), MLA's non-absorbed prefill and RoPE.

The computation lives in the HIP library libattn_gfx950.so (C ABI in include/attn.h);
``lib`` is a thin ctypes binding with the same entry points.
"""
from .lib import (  # noqa: F401
    ATTN_BF16,
    ATTN_F32,
    AttnError,
    decode,
    decode_noalloc,
    decode_noalloc_max_bytes,
    decode_workspace_bytes,
    kernel_events,
    kv_append,
    load,
    prefill,
    prefill_cached,
    prefill_cached_workspace_bytes,
    prefill_mla,
    prefill_mla_workspace_bytes,
    prefill_workspace_bytes,
    rope_apply_,
    status_str,
)
