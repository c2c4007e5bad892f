"""Build checks of the HIP library that need no GPU.

The decode kernels are sized to the 128 registers a lane has at 16 waves
per workgroup; a change that makes one of them spill to scratch memory
still computes the right result but slows the kernel down by microseconds
(a bf16 tail's masking select once cost 148 bytes per lane and +3.3 us at
32K).  The compiler's resource remarks name the scratch size of every
kernel; this test requires zero for each.
"""
import os
import re
import shutil
import subprocess

import pytest

from kv_cache_int2_fwht_amd import build as obuild

KERNELS = ("decode_int2_kernel", "decode_bf16_kernel", "merge_splits_kernel", "quantize_kv_kernel")


def _hipcc():
    try:
        return obuild.hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not installed")
def test_kernels_use_no_scratch(tmp_path):
    flags = [f for f in obuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    seen = {}
    for src in obuild.sources():
        cmd = [_hipcc(), *flags, "--offload-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
               "-o", str(tmp_path / (os.path.basename(src) + ".o")), src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        name = None
        for line in res.stderr.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                continue
            m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
            if m and name is not None:
                seen[name] = int(m.group(1))
                name = None
    for k in KERNELS:
        assert any(k in n for n in seen), f"no resource remark for {k}"
    spills = {n: s for n, s in seen.items() if s != 0}
    assert not spills, f"kernels with scratch (register spills): {spills}"
