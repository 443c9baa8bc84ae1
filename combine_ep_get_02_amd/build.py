"""Build libep.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m combine_ep_get_02_amd.build

The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIBRARY = os.path.join(PKG, "libep.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fused multiply-add in the kernels is written out (fmaf); nothing else is contracted
    "-ffp-contract=off",
    # no packed-fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def build(out: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = ["hipcc", *FLAGS, *(extra or []), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
