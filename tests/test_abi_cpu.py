"""The C ABI library on the host: it loads, exports every function that
include/oscar.h declares, and validates arguments before touching a device.

Tests that pass placeholder pointers run only where no GPU is present: there
the library must stop at validation (or report that no device exists)
without launching anything.
"""
import ctypes
import os
import re

import pytest

from kv_cache_int2_fwht_amd import binding as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    L = ob.lib()
    declared = _declared_functions()
    assert len(declared) >= 7
    for name in declared:
        assert hasattr(L, name), f"{name} declared in oscar.h but not exported"
    assert set(declared) == set(ob.EXPORTED)


def test_probe_library_exports_every_declared_function():
    from kv_cache_int2_fwht_amd import probes
    text = open(os.path.join(ROOT, "include", "oscar_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text)))
    assert set(declared) == set(probes.EXPORTED)
    L = probes.lib()
    for name in declared:
        assert hasattr(L, name), f"{name} declared in oscar_probe.h but not exported"
    # invalid arguments are refused before any launch
    assert L.oscar_probe_stream(0, 1, 8, 1024, 32, 0x1000, None) == 1
    assert L.oscar_probe_stream(0x10000, 1, 8, 1000, 32, 0x1000, None) == 1
    assert L.oscar_probe_clock(0, 256, 100, None) == 1


def test_version_and_status_strings():
    assert ob.abi_version() == 3
    assert ob.status_string(0) == "ok"
    assert ob.status_string(3) == "workspace too small"
    assert ob.status_string(99) == "unknown status"


def test_workspace_size_rules():
    f = ob.decode_workspace_bytes
    assert f(0, 8, 32, 1024) == 0
    assert f(1, 8, 30, 1024) == 0          # 30 query heads over 8 KV heads
    assert f(1, 8, 32, -1) == 0
    small, big = f(1, 8, 32, 8192), f(1, 8, 32, 131072)
    assert 0 < small <= big
    assert f(1, 8, 32, 0) > 0              # an empty cache still gets one (empty) split
    # one 528-byte partial record per (sequence, query head, split) at least
    assert f(8, 8, 32, 131072) >= 8 * 32 * 528
    for B, H, Hq, T in [(1, 8, 32, 131072), (8, 8, 32, 131072), (1, 1, 4, 1024), (3, 2, 16, 5000)]:
        S = ob.decode_num_splits(B, H, T)
        assert S >= 1
        assert f(B, H, Hq, T) >= B * Hq * S * 528
    assert ob.decode_num_splits(0, 8, 1024) == 0
    assert ob.decode_num_splits(1, 8, -1) == 0


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


needs_no_gpu = pytest.mark.skipif(not _no_gpu(), reason="placeholder pointers are only passed where no GPU exists")


def _desc(**kw):
    d = dict(batch=1, num_kv_heads=8, head_dim=128, group=128, capacity=1024, flags=0,
             blocks=0x10000, k_tail=0x60000, v_tail=0x70000, block_table=0, num_pages=0, reserved=0)
    d.update(kw)
    return ob.KVCacheDesc(*[d[f] for f, _ in ob.KVCacheDesc._fields_])


def _decode(desc, hq=32, max_tokens=1024, ws_bytes=1 << 26, q=0x80000, out=0x90000, ws=0xA0000):
    L = ob.lib()
    return L.oscar_decode_attn(ctypes.byref(desc) if desc is not None else None, 0x100, 0x200, max_tokens, q, hq,
                               0.088, out, ws, ws_bytes, None)


@needs_no_gpu
def test_decode_append_validation_errors():
    L = ob.lib()

    def app(desc, k_new=0xB0000, v_new=0xC0000):
        return L.oscar_decode_attn_append(ctypes.byref(desc), 0x100, 0x200, 1024, 0x80000, k_new, v_new, 32, 0.088,
                                          0x90000, 0xA0000, 1 << 26, None)
    assert app(_desc(), k_new=0) == ob.OSCAR_EINVAL
    assert app(_desc(), v_new=0xC0008) == ob.OSCAR_EINVAL        # not 16-byte aligned
    assert app(_desc(k_tail=0)) == ob.OSCAR_EINVAL                # nothing to append to
    assert b"tail" in L.oscar_last_error()
    assert app(_desc()) == ob.OSCAR_EHIP                          # valid, but no device here


@needs_no_gpu
def test_decode_validation_errors():
    L = ob.lib()
    assert _decode(None) == ob.OSCAR_EINVAL
    assert b"NULL" in L.oscar_last_error()
    assert _decode(_desc(head_dim=64)) == ob.OSCAR_EUNSUPPORTED
    assert _decode(_desc(group=64)) == ob.OSCAR_EUNSUPPORTED
    assert _decode(_desc(capacity=1000)) == ob.OSCAR_EINVAL
    assert _decode(_desc(blocks=0)) == ob.OSCAR_EINVAL
    assert _decode(_desc(blocks=0x10080)) == ob.OSCAR_EINVAL        # blocks not 256-byte aligned
    assert b"256-byte" in L.oscar_last_error()
    assert _decode(_desc(k_tail=0x60008)) == ob.OSCAR_EINVAL        # tail not 16-byte aligned
    assert _decode(_desc(flags=4)) == ob.OSCAR_EINVAL                # unknown key-variant bit
    assert b"flags" in L.oscar_last_error()
    assert _decode(_desc(), hq=30) == ob.OSCAR_EUNSUPPORTED           # not a multiple of 8 KV heads
    assert _decode(_desc(), hq=24) == ob.OSCAR_EUNSUPPORTED           # 3 query heads per KV head
    assert _decode(_desc(), max_tokens=-1) == ob.OSCAR_EINVAL
    assert _decode(_desc(), max_tokens=1024 + 128) == ob.OSCAR_EINVAL  # beyond capacity + 127
    assert _decode(_desc(), ws_bytes=64) == ob.OSCAR_EWORKSPACE
    assert b"workspace" in L.oscar_last_error()
    assert _decode(_desc(), q=0x80004) == ob.OSCAR_EINVAL


def test_cache_descriptor_mirrors_the_header():
    """The ctypes mirror has the fields of struct oscar_kv_cache, in order."""
    import re
    text = open(os.path.join(ROOT, "include", "oscar.h")).read()
    body = re.search(r"typedef struct oscar_kv_cache \{(.*?)\} oscar_kv_cache;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"(\w+)\s*;", body)
    assert names == [f for f, _ in ob.KVCacheDesc._fields_]
    assert ctypes.sizeof(ob.KVCacheDesc) == 6 * 4 + 3 * 8 + 8 + 2 * 4


@needs_no_gpu
def test_paged_descriptor_validation():
    L = ob.lib()
    assert _decode(_desc(block_table=0x50000, num_pages=0)) == ob.OSCAR_EINVAL    # a pool needs pages
    assert b"num_pages" in L.oscar_last_error()
    assert _decode(_desc(block_table=0x50002, num_pages=8)) == ob.OSCAR_EINVAL    # table not 4-byte aligned
    assert _decode(_desc(reserved=1)) == ob.OSCAR_EINVAL
    assert b"reserved" in L.oscar_last_error()
    assert _decode(_desc(block_table=0x50000, num_pages=8)) == ob.OSCAR_EHIP       # valid, but no device here
    q = L.oscar_quantize_kv(ctypes.byref(_desc(block_table=0x50000, num_pages=-1)), 0x80000, 0x90000, 0, 0, 128,
                            0x100, 0x200, 1, None)
    assert q == ob.OSCAR_EINVAL


@needs_no_gpu
def test_valid_call_without_device_reports_hip_error():
    assert _decode(_desc()) == ob.OSCAR_EHIP
    assert b"no HIP device" in ob.lib().oscar_last_error()


@needs_no_gpu
def test_splits_and_merge_validation_errors():
    L = ob.lib()

    def sp(desc, ws=0xA0000, ws_bytes=1 << 26, q=0x80000):
        return L.oscar_decode_attn_splits(ctypes.byref(desc), 0x100, 0x200, 1024, q, 32, 0.088, ws, ws_bytes, None)

    assert sp(_desc(), ws=0) == ob.OSCAR_EINVAL
    assert sp(_desc(), q=0x80002) == ob.OSCAR_EINVAL
    assert sp(_desc(), ws_bytes=100) == ob.OSCAR_EWORKSPACE
    assert sp(_desc(head_dim=96)) == ob.OSCAR_EUNSUPPORTED
    assert sp(_desc()) == ob.OSCAR_EHIP

    def mg(p=0x10000, B=1, Hq=32, S=4, out=0x20000):
        return L.oscar_decode_merge(p, B, Hq, S, out, None)

    assert mg(p=0) == ob.OSCAR_EINVAL
    assert mg(out=0x20008) == ob.OSCAR_EINVAL
    assert mg(B=0) == ob.OSCAR_EINVAL
    assert mg(B=65536) == ob.OSCAR_EINVAL
    assert mg(S=0) == ob.OSCAR_EINVAL
    assert mg() == ob.OSCAR_EHIP


@needs_no_gpu
def test_quantize_validation_errors():
    L = ob.lib()

    def q(desc, k=0xB0000, v=0xC0000, sb=8 * 1024 * 128, sh=1024 * 128, st=128, starts=0x100, ng=0x200, mg=8):
        return L.oscar_quantize_kv(ctypes.byref(desc), k, v, sb, sh, st, starts, ng, mg, None)

    assert q(_desc(), k=0) == ob.OSCAR_EINVAL
    assert q(_desc(), k=0xB0002) == ob.OSCAR_EINVAL
    assert q(_desc(), st=64) == ob.OSCAR_EINVAL
    assert q(_desc(), st=132) == ob.OSCAR_EINVAL          # not a multiple of 8 elements
    assert q(_desc(), mg=-1) == ob.OSCAR_EINVAL
    assert q(_desc(), mg=9) == ob.OSCAR_EINVAL            # more groups than the cache holds
    assert q(_desc(), mg=0) == ob.OSCAR_OK                # nothing to do
    assert q(_desc(head_dim=256)) == ob.OSCAR_EUNSUPPORTED
    assert q(_desc()) == ob.OSCAR_EHIP                    # valid, but no device here


@needs_no_gpu
def test_bf16_validation_errors():
    L = ob.lib()

    def d(k=0x10000, v=0x20000, B=1, H=8, C=1024, hq=32, mt=1024, ws_bytes=1 << 26):
        return L.oscar_decode_attn_bf16(k, v, B, H, C, 0x100, mt, 0x30000, hq, 0.088, 0x40000, 0x50000,
                                        ws_bytes, None)

    assert d(k=0) == ob.OSCAR_EINVAL
    assert d(B=0) == ob.OSCAR_EINVAL
    assert d(hq=12) == ob.OSCAR_EUNSUPPORTED
    assert d(mt=2048) == ob.OSCAR_EINVAL
    assert d(ws_bytes=10) == ob.OSCAR_EWORKSPACE
    assert d() == ob.OSCAR_EHIP


def test_noalloc_refuses_shapes_beyond_its_scratch_array():
    """oscar_decode_attn_noalloc checks the record size against its fixed
    array before anything else, GPU or not: 1024 sequences of 64 query heads
    need 1024 * 64 * 528 bytes, more than 4 MiB."""
    L = ob.lib()
    need = ob.decode_workspace_bytes(1024, 8, 64, 1024)
    assert need > ob.NOALLOC_SCRATCH_BYTES
    st = L.oscar_decode_attn_noalloc(ctypes.byref(_desc(batch=1024)), 0x100, 0x200, 1024, 0x80000, 64, 0.088,
                                     0x90000, None)
    assert st == 3
    assert b"scratch" in L.oscar_last_error()
    # the 128K layer (32 splits of 32 query heads) and batch 8 fit
    assert ob.decode_workspace_bytes(1, 8, 32, 131072) <= ob.NOALLOC_SCRATCH_BYTES
    assert ob.decode_workspace_bytes(8, 8, 32, 131072) <= ob.NOALLOC_SCRATCH_BYTES


@needs_no_gpu
def test_noalloc_validation_without_a_device():
    L = ob.lib()
    st = L.oscar_decode_attn_noalloc(ctypes.byref(_desc(head_dim=64)), 0x100, 0x200, 1024, 0x80000, 32, 0.088,
                                     0x90000, None)
    assert st == 2
    st = L.oscar_decode_attn_noalloc(ctypes.byref(_desc()), 0x100, 0x200, 1024, 0x80000, 32, 0.088, 0x90000, None)
    assert st == 4 and b"no HIP device" in L.oscar_last_error()
