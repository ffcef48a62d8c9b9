"""Builds libmla_decode.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mla_decode.hip")
SOURCES = [SRC, os.path.join(HERE, "csrc", "mla_combine.hip"), os.path.join(HERE, "csrc", "mla_topk.hip")]
HEADER = os.path.join(ROOT, "include", "mla_decode.h")
LIB = os.path.join(HERE, "libmla_decode.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(force: bool = True) -> str:
    """Compile the library (always, unless force=False and it is newer than its sources)."""
    if not force and os.path.exists(LIB):
        newest = max(max(os.path.getmtime(f) for f in SOURCES), os.path.getmtime(HEADER),
                     os.path.getmtime(__file__))
        if os.path.getmtime(LIB) >= newest:
            return LIB
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
