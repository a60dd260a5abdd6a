"""Build liblnr.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m layernorm_reduction_amd.build
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
LIB = os.path.join(PKG, "liblnr.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        # No packed-fp32 instructions: hipcc emits plain VALU fp32 ops instead.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), *flags(), *sources(), "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


C_CLIENT_SRC = os.path.join(ROOT, "tests", "native", "c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "native", "c_client")


def build_c_client(verbose: bool = False) -> str:
    """The plain C99 client of the C ABI (tests/native/c_client.c), compiled by the host C
    compiler against include/lnr.h, liblnr.so and the HIP runtime; no device code."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [os.environ.get("CC", "gcc"), "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{INCLUDE}", f"-I{rocm}/include", C_CLIENT_SRC, "-o", C_CLIENT + ".tmp", f"-L{PKG}", "-llnr",
           f"-L{rocm}/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{rocm}/lib",
           "-Wl,-rpath,$ORIGIN/../../layernorm_reduction_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(C_CLIENT + ".tmp", C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
    print(build_c_client(verbose="-q" not in sys.argv))
