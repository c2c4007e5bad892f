"""OScaR INT2 KV cache for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``_lib/liboscar.so`` (C ABI in
``include/oscar.h``); ``binding`` marshals torch tensors into it.
"""
from . import binding  # noqa: F401
from .binding import (PackedCache, OscarError, quantize_kv, decode_attn, decode_attn_append, decode_attn_bf16,  # noqa: F401
                      decode_attn_noalloc, decode_workspace_bytes, alloc_workspace, decode_num_splits,
                      decode_attn_splits, decode_merge, split_records)
from .session import DecodeSession, plan_steps  # noqa: F401

__all__ = ["binding", "PackedCache", "OscarError", "quantize_kv", "decode_attn", "decode_attn_append",
           "decode_attn_bf16", "decode_attn_noalloc", "decode_workspace_bytes", "alloc_workspace",
           "decode_num_splits", "decode_attn_splits", "decode_merge", "split_records", "DecodeSession", "plan_steps"]
