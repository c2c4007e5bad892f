"""ctypes loader of the measurement probes (``_lib/liboscar_probe.so``,
declared in ``include/oscar_probe.h``): the decode kernel's cache stream
without compute, and a shader-clock probe.  Used by the benchmark only."""
from __future__ import annotations

import ctypes
import os

_LIB = None
EXPORTED = ("oscar_probe_stream", "oscar_probe_clock", "oscar_probe_wall_clock_khz")


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "liboscar_probe.so")


def lib():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with python -m kv_cache_int2_fwht_amd.build")
        L = ctypes.CDLL(path)
        i32, vp = ctypes.c_int32, ctypes.c_void_p
        L.oscar_probe_stream.restype = i32
        L.oscar_probe_stream.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oscar_probe_clock.restype = i32
        L.oscar_probe_clock.argtypes = [vp, i32, i32, vp]
        L.oscar_probe_wall_clock_khz.restype = i32
        L.oscar_probe_wall_clock_khz.argtypes = []
        _LIB = L
    return _LIB
