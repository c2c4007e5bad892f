"""ctypes binding of the C ABI in ``include/oscar.h`` (argument marshalling only).

Every function here has the same name as its C entry point without the
``oscar_`` prefix.  Tensors are torch tensors on the GPU; this module checks
dtypes, shapes, contiguity and devices, turns them into pointers and passes
torch's current stream.  All computation happens in the HIP library; if the
library is missing this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HEAD_DIM = 128
GROUP = 128
# one group's block in the packed cache (byte offsets; include/oscar.h)
BLOCK_K_CODES, BLOCK_V_CODES, BLOCK_K_SZ, BLOCK_V_SZ, BLOCK_K_NORM = 0, 4096, 8192, 8704, 9216
BLOCK_BYTES = 9472
# oscar_kv_cache.flags: key-quantizer variants (Token Norm Imbalance ablation)
KEYS_UNROTATED, KEYS_UNSCALED = 1, 2

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "liboscar.so")
_lib = None

OSCAR_OK, OSCAR_EINVAL, OSCAR_EUNSUPPORTED, OSCAR_EWORKSPACE, OSCAR_EHIP = range(5)


class OscarError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"oscar status {status}: {message}")
        self.status = status


class KVCacheDesc(ctypes.Structure):
    """Mirror of ``struct oscar_kv_cache``."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("blocks", ctypes.c_void_p),
        ("k_tail", ctypes.c_void_p),
        ("v_tail", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


EXPORTED = (
    "oscar_abi_version", "oscar_status_string", "oscar_last_error",
    "oscar_quantize_kv", "oscar_decode_workspace_bytes",
    "oscar_decode_attn", "oscar_decode_attn_append", "oscar_decode_attn_bf16",
    "oscar_decode_num_splits", "oscar_decode_attn_splits", "oscar_decode_merge",
    "oscar_decode_attn_noalloc",
)


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                           "(run __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.oscar_abi_version.restype = i32
    L.oscar_abi_version.argtypes = []
    L.oscar_status_string.restype = ctypes.c_char_p
    L.oscar_status_string.argtypes = [ctypes.c_int]
    L.oscar_last_error.restype = ctypes.c_char_p
    L.oscar_last_error.argtypes = []
    L.oscar_quantize_kv.restype = ctypes.c_int
    L.oscar_quantize_kv.argtypes = [ctypes.POINTER(KVCacheDesc), vp, vp, i64, i64, i64, vp, vp, i32, vp]
    L.oscar_decode_workspace_bytes.restype = sz
    L.oscar_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.oscar_decode_attn.restype = ctypes.c_int
    L.oscar_decode_attn.argtypes = [ctypes.POINTER(KVCacheDesc), vp, vp, i32, vp, i32, f32, vp, vp, sz, vp]
    L.oscar_decode_attn_append.restype = ctypes.c_int
    L.oscar_decode_attn_append.argtypes = [ctypes.POINTER(KVCacheDesc), vp, vp, i32, vp, vp, vp, i32, f32, vp, vp,
                                           sz, vp]
    L.oscar_decode_attn_bf16.restype = ctypes.c_int
    L.oscar_decode_attn_bf16.argtypes = [vp, vp, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]
    L.oscar_decode_num_splits.restype = i32
    L.oscar_decode_num_splits.argtypes = [i32, i32, i32]
    L.oscar_decode_attn_splits.restype = ctypes.c_int
    L.oscar_decode_attn_splits.argtypes = [ctypes.POINTER(KVCacheDesc), vp, vp, i32, vp, i32, f32, vp, sz, vp]
    L.oscar_decode_attn_noalloc.restype = ctypes.c_int
    L.oscar_decode_attn_noalloc.argtypes = [ctypes.POINTER(KVCacheDesc), vp, vp, i32, vp, i32, f32, vp, vp]
    L.oscar_decode_merge.restype = ctypes.c_int
    L.oscar_decode_merge.argtypes = [vp, i32, i32, i32, vp, vp]
    _lib = L
    return L


def _check(status: int):
    if status != OSCAR_OK:
        msg = lib().oscar_last_error().decode(errors="replace")
        raise OscarError(status, msg)


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype, name: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def abi_version() -> int:
    return lib().oscar_abi_version()


def status_string(status: int) -> str:
    return lib().oscar_status_string(status).decode()


def last_error() -> str:
    return lib().oscar_last_error().decode(errors="replace")


class PackedCache:
    """Caller-owned packed cache (torch tensors) and its descriptor.

    ``blocks`` is uint8 [B, H, C/128, 9472] (B = batch, H = KV heads,
    C = capacity): one block per group of 128 tokens.  The fields are views
    into it, one group per index of dimension 2:
      k_codes uint8 [B,H,G,128,32]   k_sz int16 [B,H,G,128,2] (fp16 bits)
      v_codes uint8 [B,H,G,128,32]   v_sz int16 [B,H,G,128,2] (fp16)
      k_norm  int16 [B,H,G,128] (fp16)
    fp16 data is viewed as int16 so that the bit patterns are exact.
    k_tail / v_tail are bf16 [B,H,128,128].

    Paged layout (``num_pages`` given): ``blocks`` is a pool uint8
    [num_pages, H, 9472], one page per group for all KV heads, and
    ``block_table`` int32 [B, C/128] (on the device) names the page of each
    group.  The default table gives sequence b's groups the pages
    b * C/128 + g; any table whose entries are pages of the pool works.
    """

    def __init__(self, batch: int, num_kv_heads: int, capacity: int, device="cuda", flags: int = 0,
                 num_pages: Optional[int] = None, block_table: Optional[torch.Tensor] = None):
        if capacity % GROUP:
            raise ValueError("capacity must be a multiple of 128")
        B, H, C = batch, num_kv_heads, capacity
        dev = torch.device(device)
        self.batch, self.num_kv_heads, self.capacity = B, H, C
        self.flags = int(flags)   # KEYS_UNROTATED | KEYS_UNSCALED; 0 = OScaR
        self.num_pages = None if num_pages is None else int(num_pages)
        self.block_table = None
        if self.num_pages is None:
            if block_table is not None:
                raise ValueError("a block table needs num_pages")
            self.blocks = torch.zeros((B, H, C // GROUP, BLOCK_BYTES), dtype=torch.uint8, device=dev)
        else:
            if self.num_pages <= 0:
                raise ValueError("num_pages must be positive")
            self.blocks = torch.zeros((self.num_pages, H, BLOCK_BYTES), dtype=torch.uint8, device=dev)
            if block_table is None:
                block_table = torch.arange(B * (C // GROUP), dtype=torch.int32).remainder(self.num_pages)
            block_table = block_table.to(device=dev, dtype=torch.int32).contiguous()
            if tuple(block_table.shape) != (B, C // GROUP):
                raise ValueError("block_table must be [batch, capacity / 128]")
            self.block_table = block_table
        self.k_tail = torch.zeros((B, H, GROUP, HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v_tail = torch.zeros((B, H, GROUP, HEAD_DIM), dtype=torch.bfloat16, device=dev)

    def group_blocks(self) -> torch.Tensor:
        """The blocks as [B, H, C/128, 9472] (for a paged cache, gathered
        through the block table: a copy)."""
        if self.block_table is None:
            return self.blocks
        return self.blocks[self.block_table.long()].permute(0, 2, 1, 3)

    def _part(self, off: int, nbytes: int, dtype, shape):
        if self.block_table is not None:
            raise ValueError("field views exist for the contiguous layout only (see group_blocks)")
        v = self.blocks[..., off:off + nbytes]
        if dtype is not torch.uint8:
            v = v.view(dtype)
        return v.view(*self.blocks.shape[:3], *shape)

    @property
    def k_codes(self) -> torch.Tensor:
        return self._part(BLOCK_K_CODES, 4096, torch.uint8, (GROUP, 32))

    @property
    def v_codes(self) -> torch.Tensor:
        return self._part(BLOCK_V_CODES, 4096, torch.uint8, (HEAD_DIM, 32))

    @property
    def k_sz(self) -> torch.Tensor:
        return self._part(BLOCK_K_SZ, 512, torch.int16, (HEAD_DIM, 2))

    @property
    def v_sz(self) -> torch.Tensor:
        return self._part(BLOCK_V_SZ, 512, torch.int16, (GROUP, 2))

    @property
    def k_norm(self) -> torch.Tensor:
        return self._part(BLOCK_K_NORM, 256, torch.int16, (GROUP,))

    def desc(self) -> KVCacheDesc:
        blocks = _ptr(self.blocks, torch.uint8, "blocks")
        if blocks % 256:
            raise ValueError("blocks must be 256-byte aligned")
        return KVCacheDesc(
            self.batch, self.num_kv_heads, HEAD_DIM, GROUP, self.capacity, self.flags, blocks,
            _ptr(self.k_tail, torch.bfloat16, "k_tail"), _ptr(self.v_tail, torch.bfloat16, "v_tail"),
            _ptr(self.block_table, torch.int32, "block_table"), self.num_pages or 0, 0)

    def nbytes_packed(self) -> int:
        """Bytes of the packed representation (codes, scales, zero-points, norms)."""
        return self.blocks.numel()


def quantize_kv(cache: PackedCache, k_src: torch.Tensor, v_src: torch.Tensor,
                dst_group_start: torch.Tensor, num_groups: torch.Tensor, max_groups: int,
                stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_quantize_kv.  k_src / v_src: bf16 [B, H, T, 128] views with unit
    channel stride (other strides arbitrary multiples of 8)."""
    for name, t in (("k_src", k_src), ("v_src", v_src)):
        if t.dim() != 4 or t.shape[0] != cache.batch or t.shape[1] != cache.num_kv_heads or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{name} must be [batch, kv_heads, tokens, 128]")
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.stride(3) != 1:
            raise ValueError(f"{name} must be a bf16 GPU tensor with unit channel stride")
    if k_src.stride() != v_src.stride():
        raise ValueError("k_src and v_src must have the same strides")
    if k_src.shape[2] < max_groups * GROUP:
        raise ValueError("source has fewer than max_groups * 128 tokens")
    d = cache.desc()
    sb, sh, st, _ = k_src.stride()
    _check(lib().oscar_quantize_kv(ctypes.byref(d), k_src.data_ptr(), v_src.data_ptr(), sb, sh, st,
                                   _ptr(dst_group_start, torch.int32, "dst_group_start"),
                                   _ptr(num_groups, torch.int32, "num_groups"), int(max_groups),
                                   _stream(stream)))


def decode_workspace_bytes(batch: int, num_kv_heads: int, num_q_heads: int, max_tokens: int) -> int:
    return int(lib().oscar_decode_workspace_bytes(batch, num_kv_heads, num_q_heads, max_tokens))


def alloc_workspace(batch: int, num_kv_heads: int, num_q_heads: int, max_tokens: int,
                    device="cuda") -> torch.Tensor:
    """A workspace (uint8) of the size the library asks for."""
    n = decode_workspace_bytes(batch, num_kv_heads, num_q_heads, max_tokens)
    if n == 0:
        raise ValueError("invalid decode shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_attn(cache: PackedCache, n_quant: torch.Tensor, n_tail: torch.Tensor, max_tokens: int,
                q: torch.Tensor, sm_scale: float, out: torch.Tensor, ws: torch.Tensor,
                stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_attn.  q bf16 [B, Hq, 128]; out fp32 [B, Hq, 128]."""
    if q.dim() != 3 or q.shape[0] != cache.batch or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, q_heads, 128]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    d = cache.desc()
    _check(lib().oscar_decode_attn(ctypes.byref(d), _ptr(n_quant, torch.int32, "n_quant"),
                                   _ptr(n_tail, torch.int32, "n_tail"), int(max_tokens),
                                   _ptr(q, torch.bfloat16, "q"), q.shape[1], float(sm_scale),
                                   _ptr(out, torch.float32, "out"), _ptr(ws, torch.uint8, "ws"),
                                   ws.numel(), _stream(stream)))


def decode_attn_append(cache: PackedCache, n_quant: torch.Tensor, n_tail: torch.Tensor, max_tokens: int,
                       q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, sm_scale: float,
                       out: torch.Tensor, ws: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_attn_append.  k_new / v_new bf16 [B, Hkv, 128] (the step's
    own key and value, stored at tail index n_tail - 1 and attended)."""
    if q.dim() != 3 or q.shape[0] != cache.batch or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, q_heads, 128]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (cache.batch, cache.num_kv_heads, HEAD_DIM):
            raise ValueError(f"{name} must be [batch, kv_heads, 128]")
    d = cache.desc()
    _check(lib().oscar_decode_attn_append(ctypes.byref(d), _ptr(n_quant, torch.int32, "n_quant"),
                                          _ptr(n_tail, torch.int32, "n_tail"), int(max_tokens),
                                          _ptr(q, torch.bfloat16, "q"), _ptr(k_new, torch.bfloat16, "k_new"),
                                          _ptr(v_new, torch.bfloat16, "v_new"), q.shape[1], float(sm_scale),
                                          _ptr(out, torch.float32, "out"), _ptr(ws, torch.uint8, "ws"),
                                          ws.numel(), _stream(stream)))


def decode_attn_bf16(k: torch.Tensor, v: torch.Tensor, seq_len: torch.Tensor, max_tokens: int,
                     q: torch.Tensor, sm_scale: float, out: torch.Tensor, ws: torch.Tensor,
                     stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_attn_bf16.  k, v bf16 [B, Hkv, capacity, 128]."""
    if k.dim() != 4 or k.shape != v.shape or k.shape[3] != HEAD_DIM:
        raise ValueError("k and v must be [batch, kv_heads, capacity, 128]")
    if q.dim() != 3 or q.shape[0] != k.shape[0] or out.shape != q.shape:
        raise ValueError("q / out must be [batch, q_heads, 128]")
    B, H, C, _ = k.shape
    _check(lib().oscar_decode_attn_bf16(_ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"), B, H, C,
                                        _ptr(seq_len, torch.int32, "seq_len"), int(max_tokens),
                                        _ptr(q, torch.bfloat16, "q"), q.shape[1], float(sm_scale),
                                        _ptr(out, torch.float32, "out"), _ptr(ws, torch.uint8, "ws"),
                                        ws.numel(), _stream(stream)))


def decode_num_splits(batch: int, num_kv_heads: int, max_tokens: int) -> int:
    """oscar_decode_num_splits: records per (sequence, query head)."""
    return int(lib().oscar_decode_num_splits(batch, num_kv_heads, max_tokens))


def decode_attn_splits(cache: PackedCache, n_quant: torch.Tensor, n_tail: torch.Tensor, max_tokens: int,
                       q: torch.Tensor, sm_scale: float, ws: torch.Tensor,
                       stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_attn_splits: the split records of one decode step,
    written at the start of ws as float [B, Hq, S, 132]."""
    if q.dim() != 3 or q.shape[0] != cache.batch or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, q_heads, 128]")
    d = cache.desc()
    _check(lib().oscar_decode_attn_splits(ctypes.byref(d), _ptr(n_quant, torch.int32, "n_quant"),
                                          _ptr(n_tail, torch.int32, "n_tail"), int(max_tokens),
                                          _ptr(q, torch.bfloat16, "q"), q.shape[1], float(sm_scale),
                                          _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))


def split_records(ws: torch.Tensor, batch: int, num_q_heads: int, num_splits: int) -> torch.Tensor:
    """View of the records at the start of a workspace: float [B, Hq, S, 132]."""
    n = batch * num_q_heads * num_splits * 132
    if ws.dtype != torch.uint8 or ws.numel() < 4 * n:
        raise ValueError("workspace too small for these records")
    return ws[:4 * n].view(torch.float32).view(batch, num_q_heads, num_splits, 132)


def decode_merge(partials: torch.Tensor, out: torch.Tensor,
                 stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_merge.  partials float [B, Hq, S, 132]; out fp32 [B, Hq, 128]."""
    if partials.dim() != 4 or partials.shape[3] != 132:
        raise ValueError("partials must be [batch, q_heads, splits, 132]")
    B, Hq, S, _ = partials.shape
    if out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be [batch, q_heads, 128]")
    _check(lib().oscar_decode_merge(_ptr(partials, torch.float32, "partials"), B, Hq, S,
                                    _ptr(out, torch.float32, "out"), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 4 << 20   # OSCAR_NOALLOC_SCRATCH_BYTES


def decode_attn_noalloc(cache: PackedCache, n_quant: torch.Tensor, n_tail: torch.Tensor, max_tokens: int,
                        q: torch.Tensor, sm_scale: float, out: torch.Tensor,
                        stream: Optional[torch.cuda.Stream] = None) -> None:
    """oscar_decode_attn_noalloc: oscar_decode_attn with the split records in
    the library's own device array (no workspace; calls on one device must
    not overlap)."""
    if q.dim() != 3 or q.shape[0] != cache.batch or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, q_heads, 128]")
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    d = cache.desc()
    _check(lib().oscar_decode_attn_noalloc(ctypes.byref(d), _ptr(n_quant, torch.int32, "n_quant"),
                                           _ptr(n_tail, torch.int32, "n_tail"), int(max_tokens),
                                           _ptr(q, torch.bfloat16, "q"), q.shape[1], float(sm_scale),
                                           _ptr(out, torch.float32, "out"), _stream(stream)))
