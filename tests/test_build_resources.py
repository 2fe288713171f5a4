"""Register budget of the forward kernels (host only: compiles for gfx950, runs nothing).

The persistent kernel sits at its register limit (256 VGPRs for two
workgroups per CU).  A change anywhere in it can tip the allocator into
spilling VGPRs to scratch, which slows the MFMA loop several times over
without any error.  This test compiles the kernel source with the compiler's
resource-usage remarks and fails when the kernels of the DeepSeek-shape calls
(128-row tiles at T=8192, 16-row wave tiles at T=128, both e4m3 x e2m1 on the
TILED weights) spill VGPRs or use scratch memory."""
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_ffn_histogram_amd import build as B

KERNELS = {
    "_ZN6moeffn14moe_ffn_kernelILi2ELi128ELb1EEEvNS_7KParamsE": "128-row tiles, e4m3 x e2m1, TILED",
    "_ZN6moeffn14moe_ffn_kernelILi2ELi16ELb1EEEvNS_7KParamsE": "16-row wave tiles, e4m3 x e2m1, TILED",
}


def _remarks() -> dict:
    out = os.path.join(B.BUILD, "resource_check.o")
    os.makedirs(B.BUILD, exist_ok=True)
    cmd = ([B.HIPCC] + B.COMMON + ["--cuda-device-only", "-x", "hip", "-c",
                                   os.path.join(B.CSRC, "moe_ffn_kernel.hip"), "-o", out,
                                   "-Rpass-analysis=kernel-resource-usage"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    usage, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            usage[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur is not None:
            usage[cur][m.group(1).strip()] = int(m.group(2))
    return usage


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_hot_kernels_do_not_spill():
    usage = _remarks()
    for name, what in KERNELS.items():
        assert name in usage, f"{what}: kernel {name} not found in the compiler's remarks"
        u = usage[name]
        assert u.get("VGPRs Spill", 0) == 0, f"{what}: {u.get('VGPRs Spill')} VGPRs spilled ({u})"
        assert u.get("ScratchSize", 0) == 0, f"{what}: {u.get('ScratchSize')} bytes of scratch per lane ({u})"
        assert u.get("Occupancy", 2) >= 2, f"{what}: occupancy {u.get('Occupancy')} < 2 waves per SIMD ({u})"
