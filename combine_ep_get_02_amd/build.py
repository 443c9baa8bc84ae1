"""Build libep.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
the plain-C example program that the GPU tests run against it.

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


C_EXAMPLE_SOURCE = os.path.join(ROOT, "tests", "c_abi_roundtrip.c")
C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi_roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_example(verbose: bool = False) -> str:
    """gcc (C11) build of tests/c_abi_roundtrip.c linked against libep.so and the
    HIP runtime, with run paths so it runs from the tree as it is."""
    # the HIP runtime headers must be told the platform when a plain C compiler reads them
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROCM, "include"), C_EXAMPLE_SOURCE, "-L", PKG, "-lep", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../combine_ep_get_02_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", C_EXAMPLE]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return C_EXAMPLE


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
    print(build_c_example(verbose=True))
    sys.exit(0)
