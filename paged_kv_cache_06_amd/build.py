"""Build libpagedattn.so in-tree with hipcc for gfx950.

Each source compiles to an object in its own hipcc process (in parallel:
the fp16-pool and E4M3-pool decode instances are the slow ones), then one
hipcc call links the shared library.
"""

from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRC = os.path.join(CSRC, "pagedattn.hip")  # decode attention: host side and fp16-pool instances
SOURCES = [
    SRC,
    os.path.join(CSRC, "pagedattn_fp8.hip"),  # E4M3-pool instances of the decode kernel
    os.path.join(CSRC, "blockops.hip"),  # the block operations
]
HEADERS = [os.path.join(CSRC, "decode_kernel.h"), os.path.join(CSRC, "e4m3.h")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpagedattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the decode kernel's accumulators are
    # also read and scaled by vector instructions, and with the default choice
    # (accumulation registers) every product was bracketed by copies in and out,
    # which serialised the eight output products of a step
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src: str, obj: str, extra) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")


def build(out: str = LIB, extra=()) -> str:
    objs = [out + "." + os.path.splitext(os.path.basename(s))[0] + ".o" for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for f in [ex.submit(_compile, s, o, tuple(extra)) for s, o in zip(SOURCES, objs)]:
            f.result()
    tmp = out + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       stderr=subprocess.PIPE, text=True)
    for o in objs:
        os.remove(o)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
