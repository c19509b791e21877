"""Build libepx.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m combine_ep_dispatch_amd.build

Flags:
  --offload-arch=gfx950                      MI355X only
  -ffp-contract=off                          no fused multiply-add: every fp32
                                             op rounds once, as the method
                                             states its arithmetic
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division for 2688/rowmax etc.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             keep the compiler from forming
                                             packed fp32 VALU ops
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libepx.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libepx.so)")


def compile_flags() -> list:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libepx.so next to this file."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in sources:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
