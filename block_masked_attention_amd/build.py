"""Build libbdattn.so (the C ABI plus its gfx950 kernels) in-tree with hipcc.

Run ``python -m block_masked_attention_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdattn.so")
SOURCES = ["api.cpp", "plan.cpp", "kernels.hip"]
HEADERS = ["bdattn_mask.h", "plan.h", "launch.h"]

# Packed fp32 ops are disabled for all device code (hipcc -O3 would otherwise
# form them from plain float code).
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the bdattn library needs ROCm's hipcc")


def build(verbose: bool = False) -> str:
    """Compile every source into libbdattn.so next to this file; return its path."""
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        # hipcc treats .cpp as host C++ unless told otherwise; api.cpp and plan.cpp
        # only launch kernels through launch.h, so compile them as HIP too.
        srcs += ["-x", "hip", p] if s.endswith(".cpp") else [p]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIP_FLAGS + ["-I", os.path.join(HERE, "..", "include")] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
