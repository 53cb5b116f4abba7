"""Builds the in-tree HIP library skinny_gemm_hcgr_amd/libhcgr.so for gfx950.

    python -m skinny_gemm_hcgr_amd.build

hipcc compiles device code for gfx950 only; packed-fp32 instructions are
disabled for device code (-Xclang -target-feature -Xclang -packed-fp32-ops);
the host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libhcgr.so")
ARCH = "gfx950"


def hipcc_command(out: str = LIB) -> list:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    return ["/opt/rocm/bin/hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), *srcs, "-o", out]


def build(out: str = LIB, verbose: bool = False) -> str:
    cmd = hipcc_command(out)
    tmp = out + ".tmp"
    cmd[-1] = tmp
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (p.stdout + p.stderr).splitlines() if noise not in ln]
    if p.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({p.returncode})")
    if verbose and msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
