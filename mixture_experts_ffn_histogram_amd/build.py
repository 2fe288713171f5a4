"""Build libmoe_ffn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_ffn.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-value"]


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in ("moe_ffn_kernel.hip", "moe_ffn_quant.hip", "moe_ffn_router.hip", "moe_ffn_noalloc.hip",
                "moe_ffn_api.cpp"):
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage and src.endswith(".hip"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd))
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        if resource_usage:
            sys.stdout.write(r.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def build_test_helpers(verbose: bool = False) -> list:
    """Compile the test-only helpers (tests/native) for gfx950: the side-stream
    kernel and the device-helper checks."""
    root = os.path.dirname(HERE)
    outs = []
    for src_name, lib_name in (("side_kernel.hip", "libmoe_side.so"), ("device_helpers.hip", "libmoe_helpers.so")):
        src = os.path.join(root, "tests", "native", src_name)
        out = os.path.join(root, "tests", "native", lib_name)
        cmd = [HIPCC] + COMMON + ["-shared", "-x", "hip", src, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd))
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on the test helper {src_name}")
        os.replace(out + ".tmp", out)
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--usage" in sys.argv))
