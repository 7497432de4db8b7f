"""Build libpagedattn.so in-tree with hipcc for gfx950."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "pagedattn.hip")  # decode attention
SOURCES = [SRC, os.path.join(HERE, "csrc", "blockops.hip")]  # and the block operations
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, *SOURCES, "-o", tmp]
    subprocess.run(cmd, check=True, stderr=subprocess.PIPE)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
