"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python moe_expert_tile_amd/build.py [--verbose]

Every call recompiles.  Device code is built with packed-fp32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["plan.hip", "gemm.hip", "combine.hip", "scale.hip", "noalloc.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def flags(resource_usage: bool = False):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
    if resource_usage:
        f += ["-Rpass-analysis=kernel-resource-usage"]
    return f


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags(resource_usage) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose or resource_usage:
        sys.stdout.write("\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resources" in sys.argv)
    print(LIB)
