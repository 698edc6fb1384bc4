"""Builds libwc.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libwc.so")
SOURCES = [os.path.join(CSRC, "wc_lib.hip"), os.path.join(CSRC, "wc_noalloc.hip")]

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # keep the compiler from forming packed FP32 ops (none are needed here)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into lossless_weight_compression_bf16_amd/libwc.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
