"""Build the HIP library ``_lib/liboscar.so`` (the OScaR path) and the
measurement probes ``_lib/liboscar_probe.so`` for gfx950 with hipcc.

Run ``python -m kv_cache_int2_fwht_amd.build`` (or ``__graft_entry__.build()``).
The library is built in-tree so that it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_lib", "liboscar.so")
PROBE_OUT = os.path.join(PKG, "_lib", "liboscar_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs (no accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(out: str, srcs, verbose: bool) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building " + os.path.basename(out))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build both libraries; returns the path of liboscar.so."""
    _compile(PROBE_OUT, sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), verbose)
    return _compile(OUT, sources(), verbose)


if __name__ == "__main__":
    print(build(verbose=True))
