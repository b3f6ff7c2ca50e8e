"""Builds libmoeroute.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m moe_token_routing_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoeroute.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # No packed-fp32 instructions in device code.  The host pass also sees
    # this feature and warns that it does not know it (harmless): hipcc's
    # -Xarch_device forwards only options without arguments, and
    # -mno-packed-fp32-ops is accepted but ignored (v_pk_fma_f32 still
    # appears), so this pair is the one spelling that works.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source in csrc/ into libmoeroute.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libmoeroute.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
