"""OScaR INT2 KV cache for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``_lib/liboscar.so`` (C ABI in
``include/oscar.h``); ``binding`` marshals torch tensors into it and
``cache.KVCache`` keeps the per-sequence lengths of a packed cache.
"""
from . import binding  # noqa: F401
from .binding import (PackedCache, OscarError, quantize_kv, decode_attn, decode_attn_bf16,  # noqa: F401
                      decode_workspace_bytes, alloc_workspace)

__all__ = ["binding", "PackedCache", "OscarError", "quantize_kv", "decode_attn",
           "decode_attn_bf16", "decode_workspace_bytes", "alloc_workspace"]
